// Grouped (prefill) forward: many tokens, each routed expert's rows batched
// into grouped GEMMs on the CDNA4 matrix cores.
//
// The pages' prefill kernel distributes per-expert tiles whose row count
// follows the routed rows, so sparse routing does not pad every expert to a
// large tile (flashinfer #4285, description: MoEDynamicKernel with tiles
// smaller than 128 rows), and reduces the routed outputs into fp32 before one
// cast (b12x #311, commit on the prefill fused-sum epilogue).  Here:
//   routing    groups the valid routes by expert (route_one, or route_zero,
//              route_count and route_place for many routes), numbers the
//              m-tiles of every expert for each GEMM (128 rows, or 32 when
//              the experts get few routes each) and records each m-tile's
//              expert and each grouped row's router weight;
//   fc1_gemm   x rows gathered into LDS, FP4 weight units copied into LDS and
//              widened to bf16 in registers (exact: E2M1 times a UE8M0 or
//              E4M3 block scale has at most 6 significant bits), v_mfma_f32_32x32x16_bf16 with
//              fp32 accumulation, SiLU(gate)*up epilogue -> the activation as
//              hi = bf16(a) plus the residual lo = a - hi: NVFP4 as two bf16
//              planes; MXFP4 as three planes (hi rounded to MXFP8, what that
//              leaves of hi, and lo as MXFP4);
//   fc2_gemm   over the activation rows and W2: NVFP4 as fc1_gemm, both bf16
//              planes on each widened weight unit (32-row m-tiles) or in two
//              passes over K, one per plane (128-row); MXFP4 in one pass on
//              v_mfma_scale_f32_32x32x64_f8f6f4, one pair per plane, block
//              and step, with the weights as stored; times the NVFP4 global and the
//              route's router weight -> fp32 rows;
//   combine    per token, the fp32 sum of its valid routes' rows in route
//              order, rounded once to bf16.
// Invalid ids (negative or >= E) join no group and are skipped by combine.
#include <hip/hip_runtime.h>

#include "act.h"
#include "decode.h"
#include "gemm_planes.h"
#include "gemm_util.h"
#include "layout.h"
#include "mxfp8.h"
#include "prefill.h"

namespace moe {

constexpr int kBK = 64;  // K elements per main-loop step (2 units)

template <typename IdT>
__device__ __forceinline__ int route_expert(const IdT* __restrict__ ids, int r, int R, int E) {
  if (r >= R) return -1;
  const int64_t v = (int64_t)ids[r];
  return (v >= 0 && v < E) ? (int)v : -1;
}

// Routing: the valid routes grouped by expert.  Expert e's routes take the
// grouped rows [grp_start[e], grp_start[e] + counts[e]) and, in each GEMM's
// m-tile numbering, its m-tiles [tile_start[e], tile_start[e + 1]); perm maps a grouped row to its route,
// rpos a route to its grouped row, and gw holds each grouped row's router
// weight.  The order of an expert's routes within
// its rows is whatever the atomics hand out: every grouped row is computed
// from its own route alone and the combine sums a token's routes in route
// order through rpos, so the layer's output does not depend on it.  Ids are
// checked before they index anything (b12x PR #311, review of dynamic.py:
// unchecked top-k ids index the per-expert counters out of bounds).
constexpr int kRouteBlock = 4096;  // routes per workgroup of the routing kernels

// Exclusive prefix over the E counters cnt (in LDS, E <= kRouteMaxExperts)
// by the 1024 threads of a workgroup: counts[e], grp_start[e] and, for each
// of the two GEMMs' m-tile sizes (FC1: bm1 rows, table ts1 / te1; FC2: bm2,
// ts2 / te2; a bm2 of 0 means FC2 shares FC1's table), tile_start[e]
// (tile_start[E] the total) and the expert of each m-tile, tile_expert[t],
// are written to global memory when `out` is set, and cnt[e] becomes
// grp_start[e].  Ends with a barrier.
__device__ void route_prefix(int* cnt, int E, int bm1, int bm2, bool out, int* __restrict__ counts,
                             int* __restrict__ grp_start, int* __restrict__ ts1, int* __restrict__ te1,
                             int* __restrict__ ts2, int* __restrict__ te2) {
  __shared__ int wpart[3][16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  constexpr int PER = kRouteMaxExperts / 1024;  // counters per thread
  const int e0 = t * PER;
  const bool two = bm2 > 0;
  if (!two) bm2 = bm1;
  int c[PER], rsum = 0, tsum1 = 0, tsum2 = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = e0 + i < E ? cnt[e0 + i] : 0;
    rsum += c[i];
    tsum1 += (c[i] + bm1 - 1) / bm1;
    tsum2 += (c[i] + bm2 - 1) / bm2;
  }
  // inclusive scans of the per-thread sums over the wave, then over the waves
  int ri = rsum, ti1 = tsum1, ti2 = tsum2;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int rv = __shfl_up(ri, m), tv1 = __shfl_up(ti1, m), tv2 = __shfl_up(ti2, m);
    if (lane >= m) {
      ri += rv;
      ti1 += tv1;
      ti2 += tv2;
    }
  }
  if (lane == 63) {
    wpart[0][wave] = ri;
    wpart[1][wave] = ti1;
    wpart[2][wave] = ti2;
  }
  __syncthreads();
  int rb = ri - rsum, tb1 = ti1 - tsum1, tb2 = ti2 - tsum2;  // exclusive within the wave
  for (int w = 0; w < wave; ++w) {
    rb += wpart[0][w];
    tb1 += wpart[1][w];
    tb2 += wpart[2][w];
  }
  int ttot1 = 0, ttot2 = 0;
  for (int w = 0; w < 16; ++w) {
    ttot1 += wpart[1][w];
    ttot2 += wpart[2][w];
  }
  __syncthreads();  // every thread has read cnt before it is overwritten
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = e0 + i;
    const int nt1 = (c[i] + bm1 - 1) / bm1, nt2 = (c[i] + bm2 - 1) / bm2;
    if (e < E) {
      if (out) {
        counts[e] = c[i];
        grp_start[e] = rb;
        ts1[e] = tb1;
        for (int q = 0; q < nt1; ++q) te1[tb1 + q] = e;
        if (two) {
          ts2[e] = tb2;
          for (int q = 0; q < nt2; ++q) te2[tb2 + q] = e;
        }
      }
      cnt[e] = rb;
    }
    rb += c[i];
    tb1 += nt1;
    tb2 += nt2;
  }
  if (out && t == 0) {
    ts1[E] = ttot1;
    if (two) ts2[E] = ttot2;
  }
  __syncthreads();
}

// All of the routing in one workgroup (R <= kRouteBlock): an LDS histogram,
// its prefix, then every route takes its grouped row from an LDS counter.
template <typename IdT>
__global__ void __launch_bounds__(1024)
    route_one(const IdT* __restrict__ ids, const float* __restrict__ tw, int R, int E, int bm1, int bm2,
              int* __restrict__ counts, int* __restrict__ grp_start, int* __restrict__ ts1,
              int* __restrict__ te1, int* __restrict__ ts2, int* __restrict__ te2, int* __restrict__ perm,
              int* __restrict__ rpos, float* __restrict__ gw) {
  __shared__ int cnt[kRouteMaxExperts];
  const int t = threadIdx.x;
  // the ids and router weights are loaded first, while the counters clear
  int ex[kRouteBlock / 1024];
  float wt[kRouteBlock / 1024];
#pragma unroll
  for (int i = 0; i < kRouteBlock / 1024; ++i) {
    const int r = t + 1024 * i;
    ex[i] = route_expert(ids, r, R, E);
    wt[i] = r < R ? tw[r] : 0.0f;
  }
  for (int q = t; q < E; q += 1024) cnt[q] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kRouteBlock / 1024; ++i)
    if (ex[i] >= 0) atomicAdd(&cnt[ex[i]], 1);
  __syncthreads();
  route_prefix(cnt, E, bm1, bm2, true, counts, grp_start, ts1, te1, ts2, te2);
#pragma unroll
  for (int i = 0; i < kRouteBlock / 1024; ++i) {
    if (ex[i] < 0) continue;
    const int r = t + 1024 * i;
    const int p = atomicAdd(&cnt[ex[i]], 1);
    perm[p] = r;
    rpos[r] = p;
    gw[p] = wt[i];
  }
}

// Routing of more routes, in three launches.  route_zero clears the
// counters; route_count adds each block's LDS histogram to counts (one
// global add per block and expert); route_place takes the prefix of
// counts, reserves each expert's range for the block (one global add per
// block and expert on fill) and hands out the rows within it from LDS.
__global__ void route_zero(int E, int* __restrict__ counts, int* __restrict__ fill) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) {
    counts[e] = 0;
    fill[e] = 0;
  }
}

template <typename IdT>
__global__ void __launch_bounds__(1024)
    route_count(const IdT* __restrict__ ids, int R, int E, int* __restrict__ counts) {
  __shared__ int cnt[kRouteMaxExperts];
  const int t = threadIdx.x;
  const int r0 = blockIdx.x * kRouteBlock;
  int ex[kRouteBlock / 1024];  // loaded while the counters clear
#pragma unroll
  for (int i = 0; i < kRouteBlock / 1024; ++i) ex[i] = route_expert(ids, r0 + t + 1024 * i, R, E);
  for (int q = t; q < E; q += 1024) cnt[q] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kRouteBlock / 1024; ++i)
    if (ex[i] >= 0) atomicAdd(&cnt[ex[i]], 1);
  __syncthreads();
  for (int q = t; q < E; q += 1024)
    if (cnt[q]) atomicAdd(&counts[q], cnt[q]);
}

template <typename IdT>
__global__ void __launch_bounds__(1024)
    route_place(const IdT* __restrict__ ids, const float* __restrict__ tw, int R, int E, int bm1, int bm2,
                int* __restrict__ counts, int* __restrict__ grp_start, int* __restrict__ ts1,
                int* __restrict__ te1, int* __restrict__ ts2, int* __restrict__ te2, int* __restrict__ fill,
                int* __restrict__ perm, int* __restrict__ rpos, float* __restrict__ gw) {
  __shared__ int cnt[kRouteMaxExperts];  // counts, then grp_start, then the block's next row per expert
  __shared__ int mine[kRouteMaxExperts];  // the block's routes per expert
  const int t = threadIdx.x;
  const int r0 = blockIdx.x * kRouteBlock;
  // the block's ids and router weights, loaded while the prefix is taken
  int ex[kRouteBlock / 1024];
  float wt[kRouteBlock / 1024];
#pragma unroll
  for (int i = 0; i < kRouteBlock / 1024; ++i) {
    const int r = r0 + t + 1024 * i;
    ex[i] = route_expert(ids, r, R, E);
    wt[i] = r < R ? tw[r] : 0.0f;
  }
  for (int q = t; q < E; q += 1024) {
    cnt[q] = counts[q];
    mine[q] = 0;
  }
  __syncthreads();
  route_prefix(cnt, E, bm1, bm2, blockIdx.x == 0, counts, grp_start, ts1, te1, ts2, te2);
#pragma unroll
  for (int i = 0; i < kRouteBlock / 1024; ++i)
    if (ex[i] >= 0) atomicAdd(&mine[ex[i]], 1);
  __syncthreads();
  for (int q = t; q < E; q += 1024)
    if (mine[q]) cnt[q] += atomicAdd(&fill[q], mine[q]);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kRouteBlock / 1024; ++i) {
    if (ex[i] < 0) continue;
    const int r = r0 + t + 1024 * i;
    const int p = atomicAdd(&cnt[ex[i]], 1);
    perm[p] = r;
    rpos[r] = p;
    gw[p] = wt[i];
  }
}

// MFMA B fragment q (K values 8q..8q+7 of a 32-value unit) from dword q of
// the unit's codes, with the block scale applied (exact: E2M1 times a UE8M0
// or E4M3 scale has at most 6 significant bits).  MXFP4: v_cvt_scalef32_pk_
// bf16_fp4 scales by the exponent of its fp32 operand, which is the UE8M0
// byte placed in the exponent field.  NVFP4: fp32 widening, times the E4M3
// scale of the 16-value half, rounded to bf16 (exact).
template <int FMT>
__device__ __forceinline__ bf16x8_t b_frag(uint32_t w, float s) {
  uint32_t o[4];
  if (FMT == kMXFP4) {
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
  } else {
    f32x2_t f[4];
    fp4x8_to_f32(w, f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x2_t b;
      b.x = (__bf16)(f[i].x * s);
      b.y = (__bf16)(f[i].y * s);
      o[i] = __builtin_bit_cast(uint32_t, b);
    }
  }
  return __builtin_bit_cast(bf16x8_t, u32x4{o[0], o[1], o[2], o[3]});
}

// Scale operand of b_frag for fragment q of unit c from the unit's scale
// dword (MXFP4: byte c % 4 as an exponent; NVFP4: E4M3 byte 2 (c % 2) + q / 2).
template <int FMT>
__device__ __forceinline__ float b_scale(uint32_t sword, int c, int q) {
  if (FMT == kMXFP4) return __uint_as_float(((sword >> (8 * (c & 3))) & 0xFFu) << 23);
  const f32x2_t sc = e4m3x2_to_f32(sword, (c & 1) != 0);
  return q < 2 ? sc.x : sc.y;
}

__device__ __forceinline__ bf16x8_t lds_frag(const __bf16* p) {
  return __builtin_bit_cast(bf16x8_t, *(const u32x4*)p);
}

// LDS of a grouped GEMM workgroup: an A ring of 3 slots x BM rows x 128
// bytes (64 bf16 per row, unpadded; the 16-byte chunk c of row r sits at
// position c ^ swz(r)), and a weight ring of 3 slots x 4 waves x (2 x 1 KiB
// codes + 256 B of scale dwords, 512 B for FC2's two passes): 75 KiB for
// FC1 with 128-row tiles (two workgroups per CU), 39 KiB with 32-row tiles.
constexpr int kARow = kBK * 2;                    // bytes of one A row of a step
template <int BM>
constexpr int kAPlane = BM * kARow;               // 16 KiB for 128 rows
// One wave's weights of a step: 2 x 1 KiB codes and the scale dwords of the
// 64 weight rows, one per row (both units of a step share it), or, for FC2's
// two passes over K (whose step can take its units from two passes), one per
// row and lane half.
template <bool PASS2>
constexpr int kBWave = 2 * 1024 + (PASS2 ? 2 : 1) * 256;
template <bool PASS2>
constexpr int kBSlot = 4 * kBWave<PASS2>;
constexpr int kBSlots = 3;
constexpr int kASlots = 3;
constexpr int kADist = kASlots - 1;  // steps ahead that A is copied (the weights: kBSlots - 1)
template <int BM, bool PASS2>
constexpr int kGemmLds = kASlots * kAPlane<BM> + kBSlots * kBSlot<PASS2>;
// With both activation planes in every step (AP = 2, one pass; 32-row
// tiles): 51 KiB, three workgroups per CU.
template <int BM>
constexpr int kGemmLds2 = kASlots * 2 * kAPlane<BM> + kBSlots * kBSlot<false>;

// Grouped GEMM main loop for one 128-row x 256-column output tile, followed
// by `epilogue(acc)`.  K runs over nU units of 32 values in steps of two; unit
// u is unit u % nC of pass u / nC (FC2 makes two passes over its K, one per
// activation plane, with the same weights).
//
// Wave w owns the 64 columns of one prepared weight tile (`btile`) and the
// first 32 * NB rows: NB x 2 MFMA 32x32x16 blocks (NB = 1..4, the 32-row
// blocks that hold rows of the tile; NB = 0 for a wave past the last weight
// tile, which only helps stage A).  Within a step the K order of the MFMAs is
// permuted so that the lanes of half h (lanes 32h..32h+31) take K values
// 32h + 8q + i in MFMA q: a lane's B operand for the four MFMAs of a step is
// then one 16-byte unit of one weight row plus its scale word, which the lane
// itself copies into its slot of the wave's weight ring two steps ahead and
// widens after reading it back; its A operand for MFMA q is the 16-byte chunk
// 4h + q of its A row.
//
// A rows (bf16, K contiguous; pass p at `plane` elements past pass 0) are
// copied into the A ring two steps ahead: wave w copies rows 32w..32w+31
// (block w), eight rows (1 KiB) per copy, from `rowp[blk]` (row
// 32w + 8 blk + lane / 8), when the tile has rows in that block (CPA; the
// A reads of a wave never go past the tile's last block).  Per step: wait
// until this wave's copies for the step have landed, one barrier, then widen
// and multiply, with the copies of A and of the weights for step s + 2
// issued between the MFMA groups (each copy occupies the address unit for a
// while; issued between MFMAs that wait hides behind them).  A copy can take
// longer to land than a step's MFMAs take to run: with A copied one step
// ahead, tiles with few rows waited for it every step.  Copies past the last step are clamped to it (never used); with an
// odd number of units the last step's second half (A and B both) is zeroed
// when read.
//
// AP = 2 (NVFP4 FC2 of 32-row tiles) takes both activation planes in one
// pass instead: a step copies and widens its weight unit once and multiplies
// it by the hi plane's fragment and the lo plane's (`plane` elements apart),
// both in the A ring's slot; PASS2 is then false.
template <int FMT, int BM, int NB, bool CPA, bool PASS2, int AP, bool NT, typename Pre, typename Epilogue>
__device__ __forceinline__ void gemm_main(const uint16_t* const (&rowp)[4], int64_t plane, int nU,
                                          const uint8_t* __restrict__ btile, int nC, uint8_t* smem, Pre&& pre,
                                          Epilogue&& epilogue) {
  static_assert(AP == 1 || (AP == 2 && !PASS2), "one or two planes per step, two only in one pass");
  constexpr int SPD = FMT == kMXFP4 ? 4 : 2;
  constexpr int NBA = NB > 0 ? NB : 1;
  // copies of later steps in flight when step s starts: those issued in the
  // steps s - kADist + 1 .. s - 1 (4 for A, 3 or 4 more for the weights)
  static_assert(kADist == kBSlots - 1, "A and the weights are copied the same number of steps ahead");
  constexpr int NW = NB > 0 ? (PASS2 ? 4 : 3) : 0;  // weight copies per step
  constexpr int BCOPIES = (kADist - 1) * ((CPA ? 4 * AP : 0) + NW);
  constexpr int ASLOT = AP * kAPlane<BM>;  // bytes of one A ring slot
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int nsteps = (nU + 1) / 2;
  const int full = nU / 2;
  uint8_t* const aring = smem;
  uint8_t* const bring = smem + kASlots * ASLOT + wave * kBWave<PASS2>;

  f32x16_t acc[NBA][2];
#pragma unroll
  for (int i = 0; i < NBA; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  // this lane's A copy source chunk (per block parity) and A read position
  const int cp_lo = (lane & 7) ^ (lane >> 3);
  const int swz = a_swz(n);
  // unit u (clamped to the last) -> byte offset in an A row
  auto a_unit = [&](int u) -> int64_t {
    u = min(u, nU - 1);
    const int p = u >= nC ? 1 : 0;
    return (int64_t)p * plane * 2 + (u - p * nC) * 64;
  };
  // copy of A rows block `blk` of plane p (AP = 2) of step s into its ring slot
  auto copy_a = [&](int s, int blk, int p) {
    const int sc = s < nsteps ? s : nsteps - 1;
    const int c = cp_lo ^ (blk & 1);
    const uint8_t* g = (const uint8_t*)rowp[blk] + p * plane * 2 + a_unit(2 * sc + (c >> 2)) + (c & 3) * 16;
    dma16(g, lds_addr(aring + (s % kASlots) * ASLOT + p * kAPlane<BM> + (32 * wave + 8 * blk) * kARow));
  };
  // chunk of this lane's weight unit in step s (clamped; within its pass)
  auto b_chunk = [&](int s) {
    const int u = min(2 * s + h, nU - 1);
    return u >= nC ? u - nC : u;
  };
  // copy of weight half j (codes and scale word) of step s into its ring slot
  auto copy_b = [&](int s, int j) {
    const int cc = b_chunk(s < nsteps ? s : nsteps - 1);
    uint8_t* slot = bring + (s % kBSlots) * kBSlot<PASS2>;
    const int row = 32 * j + n;
    if constexpr (NT)
      dma16_nt(btile + (int64_t)cc * 1024 + row * 16, lds_addr(slot + j * 1024));
    else
      dma16(btile + (int64_t)cc * 1024 + row * 16, lds_addr(slot + j * 1024));
    if constexpr (PASS2)
      dma4(btile + (int64_t)nC * 1024 + (cc / SPD) * 256 + row * 4, lds_addr(slot + 2048 + j * 256));
  };
  // the scale dwords of the step's units for the 64 weight rows (lane l: row
  // l; one pass, so both units of the step are in the same dword)
  auto copy_bs = [&](int s) {
    const int cw = min(2 * (s < nsteps ? s : nsteps - 1), nU - 1);
    dma4(btile + (int64_t)nC * 1024 + (cw / SPD) * 256 + lane * 4,
         lds_addr(bring + (s % kBSlots) * kBSlot<PASS2> + 2048));
  };
  // Copies of a step, always issued in this order (vm_wait counts on it):
  // copies 0..4AP-1 are A blocks for step s + 2 (none without CPA), then the
  // weight halves for the same step and (one pass) their scales.
  constexpr int NCA = 4 * AP;
  constexpr int NCOPY = NB > 0 ? NCA + (PASS2 ? 2 : 3) : NCA;
  constexpr int NGROUP = 4 * NB;                             // MFMA groups of a step
  constexpr int NPRE = NCOPY > NGROUP ? NCOPY - NGROUP : 0;  // copies issued before them
  auto copy = [&](int s, int ci) {
    if (ci < NCA) {
      if constexpr (CPA) copy_a(s + kADist, ci & 3, ci >> 2);
    } else if (ci < NCA + 2) {
      copy_b(s + kADist, ci - NCA);
    } else {
      copy_bs(s + kADist);
    }
  };
  auto widen = [&](int s, bool tail, bf16x8_t (&bf)[4][2]) {
    const uint8_t* slot = bring + (s % kBSlots) * kBSlot<PASS2>;
    const int c = b_chunk(s);
    const bool z = tail && h;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4 w = *(const u32x4*)(slot + j * 1024 + lane * 16);
      const uint32_t sw = *(const uint32_t*)(slot + 2048 + (PASS2 ? j * 256 + lane * 4 : (32 * j + n) * 4));
#pragma unroll
      for (int q = 0; q < 4; ++q) bf[q][j] = z ? bf16x8_t{} : b_frag<FMT>(w[q], b_scale<FMT>(sw, c, q));
    }
  };
  auto mfmas = [&](int s, bool tail, const bf16x8_t (&bf)[4][2]) {
    const uint8_t* slot = aring + (s % kASlots) * ASLOT;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
#pragma unroll
        for (int p = 0; p < AP; ++p) {
          bf16x8_t af = lds_frag(
              (const __bf16*)(slot + p * kAPlane<BM> + (i * 32 + n) * kARow + (((4 * h + q) ^ swz) * 16)));
          if (tail && h) af = bf16x8_t{};
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[q][j], acc[i][j], 0, 0, 0);
        }
        // one of this step's copies after each of the first MFMA groups
        const int ci = NPRE + q * NB + i;
        if (ci < NCOPY) copy(s, ci);
      }
    }
  };
  auto step = [&](int s, bool tail) {
    vm_wait<BCOPIES>();  // this wave's copies of A(s) and B(s) have landed
    __syncthreads();     // everyone's A(s) has; everyone is done with step s - 1
#pragma unroll
    for (int ci = 0; ci < NPRE; ++ci) copy(s, ci);
    if constexpr (NB > 0) {
      bf16x8_t bf[4][2];
      widen(s, tail, bf);
      mfmas(s, tail, bf);
    }
  };

  // the first kADist steps' copies, step by step in the same order
#pragma unroll
  for (int s = 0; s < kADist; ++s) {
    if constexpr (CPA) {
#pragma unroll
      for (int p = 0; p < AP; ++p)
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) copy_a(s, blk, p);
    }
    if constexpr (NB > 0) {
      copy_b(s, 0);
      copy_b(s, 1);
      if constexpr (!PASS2) copy_bs(s);
    }
  }
  for (int s = 0; s < full; ++s) step(s, false);
  if (full < nsteps) step(full, true);
  pre();             // LDS the epilogue reads, written before the barrier
  vm_wait<0>();      // no copy may land after the workgroup's LDS is released
  __syncthreads();
  if constexpr (NB > 0) epilogue(acc);
}

// gemm_main with NB = the number of 32-row blocks holding the tile's rows
// (0 when the wave has no weight tile); the wave copies its A block when the
// tile has rows in it.  Tiles of BM = 32 rows have one block, copied by wave
// 0.  Each variant carries its own copy of the epilogue, called with the
// NB x 2 accumulator blocks.
template <int FMT, int BM, bool PASS2, int AP, bool NT, typename Pre, typename Epilogue>
__device__ __forceinline__ void gemm_rows(int rows, const uint16_t* const (&rowp)[4], int64_t plane, int nU,
                                          const uint8_t* __restrict__ btile, bool bok, int nC,
                                          uint8_t* smem, Pre&& pre, Epilogue&& ep) {
  const bool cpa = 32 * (threadIdx.x >> 6) < rows;
  if constexpr (BM == 32) {
    if (!bok) {
      if (cpa)
        gemm_main<FMT, BM, 0, true, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
      else
        gemm_main<FMT, BM, 0, false, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
    } else {
      if (cpa)
        gemm_main<FMT, BM, 1, true, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
      else
        gemm_main<FMT, BM, 1, false, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
    }
  } else if (!bok) {
    if (cpa)
      gemm_main<FMT, BM, 0, true, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
    else
      gemm_main<FMT, BM, 0, false, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
  } else if (rows > 96) {
    gemm_main<FMT, BM, 4, true, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
  } else if (rows > 64) {
    if (cpa)
      gemm_main<FMT, BM, 3, true, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
    else
      gemm_main<FMT, BM, 3, false, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
  } else if (rows > 32) {
    if (cpa)
      gemm_main<FMT, BM, 2, true, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
    else
      gemm_main<FMT, BM, 2, false, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
  } else {
    if (cpa)
      gemm_main<FMT, BM, 1, true, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
    else
      gemm_main<FMT, BM, 1, false, PASS2, AP, NT>(rowp, plane, nU, btile, nC, smem, pre, ep);
  }
}

// bf16(v) as a float (round to nearest even).
__device__ __forceinline__ float bf16_value(float v) { return __uint_as_float((uint32_t)f32_to_bf16_rne(v) << 16); }

// One plane of an MXFP8 block of 32 values held 16 per lane by lanes 2r and
// 2r + 1: returns the block's scale byte and sets this lane's 16 codes (w,
// four to a dword in value order).  The shared exponent is the OCP one,
// raised by one where that would cap the block's largest value at 448, so
// that every value is rounded to nearest and none is clamped.  A block
// holding a NaN or an infinity gets scale byte 255 and codes 0x7F.  With
// `keep`, v becomes what the plane leaves of it (exact: a value and its
// rounding are within a factor of two); a non-finite block is left as it
// is, so the next plane is non-finite too.
__device__ __forceinline__ uint32_t mx_block16(float (&v)[16], uint32_t (&w)[4], bool keep) {
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) m = max(m, __float_as_uint(v[q]) & 0x7FFFFFFFu);
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  uint32_t sb = mx_scale_byte(m);
  if (sb == 255u) {
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = 0x7F7F7F7Fu;
    return sb;
  }
  if (__uint_as_float(m) * mx_inv_scale(sb) > 448.0f) ++sb;
  const float inv = mx_inv_scale(sb);
  const float sc = __uint_as_float(sb ? sb << 23 : 0x00400000u);  // 2^(sb - 127)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = v[4 * q + e] * inv;
    // v_cvt_pk_fp8_f32: two values to E4M3, rounded to nearest even (|x| <= 448)
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], word, true);
    w[q] = (uint32_t)word;
    if (keep) {
      v[4 * q] = (x[0] - __builtin_amdgcn_cvt_f32_fp8(word, 0)) * sc;
      v[4 * q + 1] = (x[1] - __builtin_amdgcn_cvt_f32_fp8(word, 1)) * sc;
      v[4 * q + 2] = (x[2] - __builtin_amdgcn_cvt_f32_fp8(word, 2)) * sc;
      v[4 * q + 3] = (x[3] - __builtin_amdgcn_cvt_f32_fp8(word, 3)) * sc;
    }
  }
  return sb;
}

// E2M1 code of v, |v| <= 6, rounded to nearest even (magnitudes 0, 0.5, 1,
// 1.5, 2, 3, 4, 6 are codes 0..7; the sign is bit 3).
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// An E2M1 block of 32 values held 16 per lane by lanes 2r and 2r + 1 (as
// mx_block16): returns the scale byte and sets this lane's 16 nibbles (w,
// eight to a dword, low nibble first).  The shared exponent is
// floor(log2(max |v|)) - 2 (2 = exponent of E2M1's largest power of two),
// raised by one where the largest value would exceed 6, so nothing is
// clamped; a non-finite block gets scale byte 255.
__device__ __forceinline__ uint32_t e2m1_block16(const float (&v)[16], uint32_t (&w)[2]) {
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) m = max(m, __float_as_uint(v[q]) & 0x7FFFFFFFu);
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  w[0] = w[1] = 0;
  if (m >= 0x7F800000u) return 255u;
  const int ef = (int)(m >> 23);
  uint32_t sb = (uint32_t)(ef > 2 ? ef - 2 : 0);
  if (__uint_as_float(m) * mx_inv_scale(sb) > 6.0f) ++sb;
  const float inv = mx_inv_scale(sb);
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) w[q] |= e2m1_code(v[8 * q + e] * inv) << (4 * e);
  return sb;
}

// Occupancy of the grouped GEMMs (waves per SIMD): tiles of 32 rows need a
// quarter of the A ring and a quarter of the accumulators, so three
// workgroups share a CU, and four for MXFP4 FC1 (39 KiB of LDS, 120 VGPRs;
// the other 32-row kernels would spill registers at four).
template <int BM>
constexpr int kGemmWaves = BM == 32 ? 3 : 2;
template <int FMT, int BM>
constexpr int kFc1Waves = BM == 32 && FMT == kMXFP4 ? 4 : kGemmWaves<BM>;

template <int FMT, int BM, bool NT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kFc1Waves<FMT, BM>)))
    fc1_gemm(const uint8_t* __restrict__ prep, const Layout L, const uint16_t* __restrict__ x, int k,
             const int* __restrict__ counts, const int* __restrict__ grp_start,
             const int* __restrict__ tile_start, const int* __restrict__ tile_expert,
             const int* __restrict__ perm,
             uint16_t* __restrict__ act, int64_t plane, uint8_t* __restrict__ aq, uint8_t* __restrict__ as,
             int ass) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kGemmLds<BM, false>];
  const GroupTile id = group_tile(fc1_blocks(L), tile_start, tile_expert, L.E);
  if (!id.ok) return;
  const int e = id.e;
  const int m0 = (id.gm - tile_start[e]) * BM;
  const int rows = min(BM, counts[e] - m0);
  const int gs = grp_start[e] + m0;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // wave w computes prepared FC1 tile b: its rows 0..31 are gate columns
  // 32b.., rows 32..63 the matching up columns
  const int b = 4 * id.nb + wave;
  const bool bok = b < L.nB1;
  // A rows this lane copies: rows 32 wave + 8 blk + lane / 8 of the tile
  // (grouped rows past the tile repeat its last row), each a token's x row
  const uint16_t* rowp[4];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const int r = min(32 * wave + 8 * blk + (lane >> 3), rows - 1);
    rowp[blk] = x + (int64_t)(perm[gs + r] / k) * L.H;
  }
  const float g13 = FMT == kNVFP4 ? ((const float*)prep)[e] : 1.0f;
  const int n = 32 * b + (lane & 31);
  // a = f(gate, up); a non-gated activation (relu2) writes both halves as
  // outputs, at columns n and Ip + n.  NVFP4: hi = bf16(a) and lo =
  // bf16(a - hi), two bf16 planes.  MXFP4: three planes (codes `aq`, plane p
  // at p * `plane` bytes; one scale dword per row and 32 columns at `as`,
  // `ass` bytes per row, byte p for plane p): plane 0 is hi = bf16(a)
  // rounded to MXFP8, plane 1 what that leaves of hi (E4M3 codes, a row of I
  // bytes), plane 2 lo = a - hi as MXFP4 (E2M1 nibbles, a row of I / 2
  // bytes).
  // Per 32-row block the values of a go to this wave's part of the (now idle)
  // A ring as 32 rows x 32 columns (row stride 144 B); lane l then takes row
  // l / 2, columns 16 (l % 2) .. + 15, whose block of 32 is its own 16 values
  // and its neighbour's, and stores its 16 codes of each plane at once.
  auto epilogue_mx = [&](auto& acc) __attribute__((always_inline)) {
    constexpr int NB = sizeof(acc) / sizeof(acc[0]);
    constexpr int kStride = 36;  // dwords per staged row
    float* st = (float*)(smem + wave * 32 * kStride * 4);
    const int rr = lane >> 1, half = lane & 1;
    with_act_kind(L.act.kind, [&](auto kind) __attribute__((always_inline)) {
      constexpr int K = decltype(kind)::value;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
#pragma unroll
        for (int jj = 0; jj < (K == kActRelu2 ? 2 : 1); ++jj) {
          const int col0 = jj ? L.Ip : 0;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            st[acc_row(r, lane) * kStride + (lane & 31)] =
                K == kActRelu2 && jj ? act_of<K>(L.act, acc[i][1][r], 0.0f)
                                     : act_of<K>(L.act, acc[i][0][r], acc[i][1][r]);
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging stores are done
          __builtin_amdgcn_wave_barrier();
          // this lane's 16 staged values: hi = bf16(a) (lo = false) or a - hi
          // (read again rather than kept, which leaves registers for the
          // 32-row tiles' four waves per SIMD)
          float v[16];
          auto take = [&](bool lo) __attribute__((always_inline)) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 f = *(const float4*)(st + rr * kStride + 16 * half + 4 * q);
              const float g[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) v[4 * q + e] = lo ? g[e] - bf16_value(g[e]) : bf16_value(g[e]);
            }
          };
          const int row = i * 32 + rr;
          const int c0 = col0 + 32 * b;
          uint8_t* dst = aq + (int64_t)(gs + row) * L.I + c0 + 16 * half;
          uint32_t w[4];
          take(false);
          const uint32_t s0 = mx_block16(v, w, true);
          if (row < rows) *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
          const uint32_t s1 = mx_block16(v, w, false);
          if (row < rows) *(uint4*)(dst + plane) = make_uint4(w[0], w[1], w[2], w[3]);
          take(true);
          uint32_t w4[2];
          const uint32_t s2 = e2m1_block16(v, w4);
          if (row < rows) {
            *(uint2*)(aq + 2 * plane + ((int64_t)(gs + row) * L.I + c0 + 16 * half) / 2) = make_uint2(w4[0], w4[1]);
            if (half == 0) *(uint32_t*)(as + (int64_t)(gs + row) * ass + c0 / 8) = s0 | (s1 << 8) | (s2 << 16);
          }
          __builtin_amdgcn_wave_barrier();  // the next block's staging stores come after these reads
          __builtin_amdgcn_s_waitcnt(0xC07F);
        }
      }
    });
  };
  auto epilogue = [&](auto& acc) __attribute__((always_inline)) {
    constexpr int NB = sizeof(acc) / sizeof(acc[0]);
    if constexpr (FMT == kMXFP4) {
      epilogue_mx(acc);
      return;
    }
    with_act_kind(L.act.kind, [&](auto kind) __attribute__((always_inline)) {
      constexpr int K = decltype(kind)::value;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const bool whole = i * 32 + 32 <= rows;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + acc_row(r, lane);
          if (!whole && row >= rows) continue;
          const float gate = acc[i][0][r] * g13;
          const float up = acc[i][1][r] * g13;
          const int64_t o = (int64_t)(gs + row) * L.I + n;
          const float a = act_of<K>(L.act, gate, up);
          const uint16_t hi = f32_to_bf16_rne(a);
          act[o] = hi;
          act[plane + o] = f32_to_bf16_rne(a - __uint_as_float((uint32_t)hi << 16));
          if constexpr (K == kActRelu2) {
            const float a2 = act_of<K>(L.act, up, 0.0f);
            const uint16_t hi2 = f32_to_bf16_rne(a2);
            act[o + L.Ip] = hi2;
            act[plane + o + L.Ip] = f32_to_bf16_rne(a2 - __uint_as_float((uint32_t)hi2 << 16));
          }
        }
      }
    });
  };
  gemm_rows<FMT, BM, false, 1, NT>(rows, rowp, 0, L.nC1, prep + fc1_tile_offset(L, e, bok ? b : 0), bok, L.nC1, smem,
                            [] {}, epilogue);
}

template <int FMT, int BM, bool NT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kGemmWaves<BM>)))
    fc2_gemm(const uint8_t* __restrict__ prep, const Layout L, const float* __restrict__ gw,
             const int* __restrict__ counts, const int* __restrict__ grp_start,
             const int* __restrict__ tile_start, const int* __restrict__ tile_expert,
             const int* __restrict__ perm,
             const uint16_t* __restrict__ act, int64_t plane, const uint8_t* __restrict__ aq,
             const uint8_t* __restrict__ as, int ass, float* __restrict__ y) {
  __shared__ __attribute__((aligned(1024)))
  uint8_t smem[FMT == kMXFP4 ? kPlLds<BM, 3, 1, true> : BM == 32 ? kGemmLds2<BM> : kGemmLds<BM, true>];
  __shared__ float wrow[BM];
  const GroupTile id = group_tile(fc2_blocks(L), tile_start, tile_expert, L.E);
  if (!id.ok) return;
  const int e = id.e;
  const int m0 = (id.gm - tile_start[e]) * BM;
  const int rows = min(BM, counts[e] - m0);
  const int gs = grp_start[e] + m0;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // wave w computes prepared FC2 tile hb: output columns 64hb..64hb+63
  const int hb = 4 * id.nb + wave;
  const bool bok = hb < L.nB2;
  // the router weights of the tile's rows, loaded now and put in LDS after
  // the main loop (no copy waits for them)
  const float wv = t < rows ? gw[gs + t] : 0.0f;
  auto pre = [&] {
    if (t < BM) wrow[t] = wv;
  };
  const float g2 = FMT == kNVFP4 ? ((const float*)prep)[L.E + e] : 1.0f;
  auto epilogue = [&](auto& acc) __attribute__((always_inline)) {
    constexpr int NB = sizeof(acc) / sizeof(acc[0]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = 64 * hb + j * 32 + (lane & 31);
      if (n >= L.H) continue;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const bool whole = i * 32 + 32 <= rows;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + acc_row(r, lane);
          if (!whole && row >= rows) continue;
          y[(int64_t)(gs + row) * L.H + n] = (acc[i][j][r] * g2) * wrow[row];
        }
      }
    }
  };
  const uint8_t* btile = prep + fc2_tile_offset(L, e, bok ? hb : 0);
  if constexpr (FMT == kMXFP4) {
    // one pass over the three planes: E4M3 codes of rows 32 wave + 16 blk +
    // lane / 4, E2M1 codes of row 32 wave + lane / 2, the scale dwords of row
    // 32 wave + lane % 32 (grouped rows past the tile repeat its last row)
    const uint8_t* prowp[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
      prowp[blk] = aq + (int64_t)(gs + min(32 * wave + 16 * blk + (lane >> 2), rows - 1)) * L.I;
    const uint8_t* lrow4 = aq + 2 * plane + (int64_t)(gs + min(32 * wave + (lane >> 1), rows - 1)) * (L.I / 2);
    const uint8_t* srow = as + (int64_t)(gs + min(32 * wave + (lane & 31), rows - 1)) * ass;
    gemm_rows_pl<BM, 3, 1, false, true, NT>(rows, prowp, plane, lrow4, srow, L.nC2, btile, bok, smem, pre,
                                             epilogue);
  } else {
    // rows 32 wave + 8 blk + lane / 8 of the tile; 32-row tiles take the hi
    // and lo activation planes in one pass (each weight unit copied and
    // widened once), larger ones in two passes over K, hi then lo
    const uint16_t* rowp[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
      rowp[blk] = act + (int64_t)(gs + min(32 * wave + 8 * blk + (lane >> 3), rows - 1)) * L.I;
    if constexpr (BM == 32)
      gemm_rows<FMT, BM, false, 2, NT>(rows, rowp, plane, L.nC2, btile, bok, L.nC2, smem, pre, epilogue);
    else
      gemm_rows<FMT, BM, true, 1, NT>(rows, rowp, plane, 2 * L.nC2, btile, bok, L.nC2, smem, pre, epilogue);
  }
}

// out[t][h] = bf16(sum over valid routes j of token t, in route order, of
// y[grouped row of (t, j)][h]); a token with no valid route gives +0.  One
// workgroup per (token, 1024 columns); the token's grouped rows go through
// LDS, then each thread keeps 8 rows' loads in flight.  Absent or invalid
// routes add +0, which leaves every partial sum (never -0, as the sum starts
// at +0) unchanged, so the result equals skipping them.
template <typename IdT>
__global__ void __launch_bounds__(256)
    combine(const IdT* __restrict__ ids, int k, int E, int H, const int* __restrict__ rpos,
            const float* __restrict__ y, uint16_t* __restrict__ out) {
  __shared__ int rows[256];
  const int tok = blockIdx.x;
  const int t = threadIdx.x;
  const int h = (blockIdx.y * 256 + t) * 4;
  const bool on = h < H;
  const int hh = on ? h : 0;
  float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j0 = 0; j0 < k; j0 += 256) {
    __syncthreads();
    if (j0 + t < k) {
      const int64_t r = (int64_t)tok * k + j0 + t;
      const int64_t id = (int64_t)ids[r];
      rows[t] = (id >= 0 && id < E) ? rpos[r] : -1;
    }
    __syncthreads();
    const int kc = min(256, k - j0);
    for (int u0 = 0; u0 < kc; u0 += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int rr = u0 + u < kc ? rows[u0 + u] : -1;
        // each row is read once: non-temporal loads (measured 14-15% faster)
        if (rr >= 0) {
          const u32x4 q = __builtin_nontemporal_load((const u32x4*)(y + (int64_t)rr * H + hh));
          v[u] = float4{__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z), __uint_as_float(q.w)};
        } else {
          v[u] = float4{0.0f, 0.0f, 0.0f, 0.0f};
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc.x += v[u].x;
        acc.y += v[u].y;
        acc.z += v[u].z;
        acc.w += v[u].w;
      }
    }
  }
  if (!on) return;
  uint2 o;
  o.x = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
  o.y = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
  *(uint2*)(out + (int64_t)tok * H + h) = o;
}

template <int FMT, typename IdT>
hipError_t launch_prefill_fmt(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                              const IdT* ids, const float* tw, uint16_t* out, uint8_t* ws,
                              const PrefillWs& W, int phases, bool a8, hipStream_t st) {
  const int R = M * k;
  int* counts = (int*)(ws + W.counts);
  int* grp_start = (int*)(ws + W.grp_start);
  int* ts1 = (int*)(ws + W.tile_start);  // FC1's m-tiles
  int* te1 = (int*)(ws + W.tile_expert);
  int* ts2 = (int*)(ws + W.tile_start2);  // FC2's
  int* te2 = (int*)(ws + W.tile_expert2);
  int* perm = (int*)(ws + W.perm);
  int* rpos = (int*)(ws + W.rpos);
  float* gw = (float*)(ws + W.gw);
  uint16_t* act = (uint16_t*)(ws + W.act);
  // NVFP4: elements from the hi plane to the lo plane; MXFP4: bytes from one
  // MXFP8 plane (aq, scale dwords as) to the next
  const int64_t plane = FMT == kMXFP4 ? W.pst : (W.aq - W.act) / 2;
  uint8_t* aq = ws + W.aq;
  uint8_t* as = ws + W.as;
  const int ass = 4 * L.nC2;  // bytes of a row's scale dwords
  float* y = (float*)(ws + W.y);
  // m-tiles of bm1 (FC1) and bm2 (FC2) rows: at most one partial tile per
  // expert beyond R / bm full ones
  const int bm1 = prefill_bm1(L, R, a8), bm2 = prefill_bm2(L, R, a8);
  const int64_t mt1 = (R + bm1 - 1) / bm1 + L.E, mt2 = (R + bm2 - 1) / bm2 + L.E;
  // Weights copied non-temporally while the experts get few routes each (an
  // expert's weights then serve about one 32-row tile and are read once;
  // measured 9-12% off FC1 at such loads, 13% slower with two tiles per
  // expert)
  const bool few = R <= (int64_t)kSparseRoutesPerExpert * L.E;
  // with one tile size FC2 reads FC1's table and the routing writes one
  const int rbm2 = bm2 == bm1 ? 0 : bm2;
  if (bm2 == bm1) {
    ts2 = ts1;
    te2 = te1;
  }
  if (phases & 5) {
    if (R <= kRouteBlock) {
      hipLaunchKernelGGL((route_one<IdT>), dim3(1), dim3(1024), 0, st, ids, tw, R, L.E, bm1, rbm2, counts,
                         grp_start, ts1, te1, ts2, te2, perm, rpos, gw);
    } else {
      int* fill = (int*)(ws + W.fill);
      const unsigned nb = (unsigned)((R + kRouteBlock - 1) / kRouteBlock);
      hipLaunchKernelGGL(route_zero, dim3((L.E + 255) / 256), dim3(256), 0, st, L.E, counts, fill);
      hipLaunchKernelGGL((route_count<IdT>), dim3(nb), dim3(1024), 0, st, ids, R, L.E, counts);
      hipLaunchKernelGGL((route_place<IdT>), dim3(nb), dim3(1024), 0, st, ids, tw, R, L.E, bm1, rbm2, counts,
                         grp_start, ts1, te1, ts2, te2, fill, perm, rpos, gw);
    }
  }
  const unsigned grid1 = grid8(mt1 * fc1_blocks(L)), grid2 = grid8(mt2 * fc2_blocks(L));
  if ((phases & 1) && a8) {
    const hipError_t err = launch_fc1_a8(L, prep, x, M, k, ws, W, bm1, ts1, te1, grid1, st);
    if (err != hipSuccess) return err;
  } else if (phases & 1) {
#define MOE_FC1(BM, NT)                                                                                       \
  hipLaunchKernelGGL((fc1_gemm<FMT, BM, NT>), dim3(grid1), dim3(256), 0, st, prep, L, x, k, (const int*)counts,    \
                     (const int*)grp_start, (const int*)ts1, (const int*)te1, (const int*)perm, act, plane, aq, \
                     as, ass)
    if (bm1 == 32 && few)
      MOE_FC1(32, true);
    else if (bm1 == 32)
      MOE_FC1(32, false);
    else
      MOE_FC1(kGemmBM, false);
#undef MOE_FC1
  }
  if ((phases & 2) && a8) {
    const hipError_t err = launch_fc2_a8(L, prep, ws, W, bm2, ts2, te2, grid2, st);
    if (err != hipSuccess) return err;
  } else if (phases & 2) {
#define MOE_FC2(BM, NT)                                                                                            \
  hipLaunchKernelGGL((fc2_gemm<FMT, BM, NT>), dim3(grid2), dim3(256), 0, st, prep, L, (const float*)gw,                 \
                     (const int*)counts, (const int*)grp_start, (const int*)ts2, (const int*)te2, (const int*)perm, \
                     (const uint16_t*)act, plane, (const uint8_t*)aq, (const uint8_t*)as, ass, y)
    if (bm2 == 32 && few)
      MOE_FC2(32, true);
    else if (bm2 == 32)
      MOE_FC2(32, false);
    else
      MOE_FC2(kGemmBM, false);
#undef MOE_FC2
  }
  if (phases & 10) {
    hipLaunchKernelGGL((combine<IdT>), dim3(M, (L.H + 1023) / 1024), dim3(256), 0, st, ids, k, L.E, L.H,
                       (const int*)rpos, (const float*)y, out);
  }
  return hipGetLastError();
}

template <typename IdT>
hipError_t launch_prefill(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                          const IdT* ids, const float* tw, uint16_t* out, uint8_t* ws,
                          const PrefillWs& W, int phases, bool a8, hipStream_t st) {
  if (L.fmt == kMXFP4)
    return launch_prefill_fmt<kMXFP4, IdT>(L, prep, x, M, k, ids, tw, out, ws, W, phases, a8, st);
  return launch_prefill_fmt<kNVFP4, IdT>(L, prep, x, M, k, ids, tw, out, ws, W, phases, false, st);
}

template hipError_t launch_prefill<int32_t>(const Layout&, const uint8_t*, const uint16_t*, int, int,
                                            const int32_t*, const float*, uint16_t*, uint8_t*,
                                            const PrefillWs&, int, bool, hipStream_t);
template hipError_t launch_prefill<int64_t>(const Layout&, const uint8_t*, const uint16_t*, int, int,
                                            const int64_t*, const float*, uint16_t*, uint8_t*,
                                            const PrefillWs&, int, bool, hipStream_t);

}  // namespace moe
