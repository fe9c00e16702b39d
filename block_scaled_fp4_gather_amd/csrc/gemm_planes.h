// Grouped GEMM main loop over MXFP8 activation planes times MXFP4 weights,
// all on the CDNA4 scaled matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4
// (A: E4M3 codes with one UE8M0 per 32 K values of a row, B: the prepared
// E2M1 units and their UE8M0 bytes as stored, fp32 accumulation).  An
// activation row is the sum of NP planes; the loop multiplies each plane by
// the same weights into the same accumulators, so the weights are copied
// once per step and never decoded.
//   NP = 3: the bf16-activation MXFP4 FC2 (hi = bf16(a) as two E4M3 planes,
//           and the residual a - hi as an E2M1 plane, LO4);
//   NP = 1: the W4A8-MX GEMMs (x rows, or the activation rows, quantised
//           once).
//
// Operand layout of the instruction (one wave, 64 lanes, K = 64 as two
// 32-value units): lane c + 32h holds B column c's unit h (32 E2M1 values in
// K order, 16 bytes) and that unit's scale; lane r + 32h holds A row r's
// bytes 16h..16h+15 of unit 0 followed by the same bytes of unit 1, and the
// scale of row r's unit h.  An E2M1 A operand is laid out as B: lane r + 32h
// holds row r's unit h (16 bytes, low nibble first).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_util.h"

namespace moe {

// LDS of a plane-loop workgroup whose A is copied AD steps ahead: an A ring
// of AD + 1 slots x NP planes x BM rows x 64 bytes (the 64 FP8 values of a
// step; the 16-byte chunk c of row r at position c ^ pl_swz(r)); an A scale
// ring of AD + 1 slots x BM / 32 waves x 256 bytes (lane n + 32h of wave w:
// the scale dword of row 32w + n for unit 2s + h); a weight ring of 3 slots
// x 4 waves x (2 x 1 KiB codes + 256 B: the scale dword of each of the 64
// weight rows, which covers both units of a step).  NP = 3 with LO4, AD = 1:
// 69 KiB for 128-row tiles (two workgroups per CU); NP = 1, 32-row tiles:
// 32 KiB (AD = 1) or 34 KiB (AD = 2), four workgroups per CU.
constexpr int kPlRow = 64;
template <int BM>
constexpr int kPlPlane = BM * kPlRow;  // 8 KiB for 128 rows
template <int BM>
constexpr int kPlPlane4 = BM * (kPlRow / 2);  // an E2M1 plane: 32 bytes per row and step
template <int BM, int NP, bool LO4>
constexpr int kPlSlot = (LO4 ? NP - 1 : NP) * kPlPlane<BM> + (LO4 ? kPlPlane4<BM> : 0);
template <int BM>
constexpr int kPlScale = BM / 32 * 256;
constexpr int kBWavePl = 2 * 1024 + 256;
constexpr int kBSlotPl = 4 * kBWavePl;
constexpr int kBSlotsPl = 3;
template <int BM, int NP, int AD, bool LO4>
constexpr int kPlLds = (AD + 1) * (kPlSlot<BM, NP, LO4> + kPlScale<BM>) + kBSlotsPl * kBSlotPl;

// Position swizzle of a 64-byte plane row: for every 8, 16 or 32 lanes that
// read one chunk each of rows n = lane % 32 (the same chunk index) the 16-byte
// units land in distinct LDS banks.
__device__ __forceinline__ int pl_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
// The same for a 32-byte E2M1 plane row (two chunks).
__device__ __forceinline__ int pl_swz4(int r) { return ((r >> 2) ^ (r >> 3) ^ (r >> 4)) & 1; }

// Main loop for one BM-row x 256-column output tile, followed by
// `epilogue(acc)`: one pass over the nU units of K in steps of two.  Wave w
// owns the 64 columns of one prepared weight tile (`btile`) and the first
// 32 * NB rows: NB x 2 blocks of 32 x 32 (NB = 0 for a wave past the last
// weight tile, which only helps stage A).  For each row block a step runs,
// per plane, two scaled MFMAs that take the weight unit of the lane's half
// (unit 2s + h) and the plane's codes.
//
// Scales of A (`srow`: this lane's row): SBYTE, one byte per unit (rows
// padded to whole dwords; the dword holding units 4q..4q+3 at byte 4q), so a
// single plane; else one dword per unit, byte p the scale of plane p.
//
// Copies (wave w, when the tile has rows in block w: CPA): the plane codes
// (16 rows of 64 bytes per copy, plane p at p * pst bytes from `prowp[blk]`,
// row 32w + 16 blk + lane / 4; with LO4 the last plane 32 rows of 32 bytes
// from `lrow4`, row 32w + lane / 2) and the scale dwords (row 32w + lane % 32,
// unit 2s + lane / 32), AD steps ahead; the wave's weights (two code halves
// and one copy of the 64 rows' scale dwords) two steps ahead, with NT
// non-temporally (weights read once).  Per step:
// wait until this wave's copies for the step have landed, one barrier, then
// the MFMAs with the next copies issued between them.  Copies past the last
// step are clamped to it (never used); with an odd number of units the last
// step's second unit is zeroed when read (codes and weights zero, scales 1).
template <int BM, int NP, int AD, bool SBYTE, bool LO4, bool NT, int NB, bool CPA, typename Pre, typename Epilogue>
__device__ __forceinline__ void gemm_main_pl(const uint8_t* const (&prowp)[2], int64_t pst, const uint8_t* lrow4,
                                             const uint8_t* srow, int nU, const uint8_t* __restrict__ btile,
                                             uint8_t* smem, Pre&& pre, Epilogue&& epilogue) {
  static_assert(NP >= 1 && NP <= 3 && (!SBYTE || NP == 1) && (!LO4 || NP > 1), "planes and their scales");
  constexpr int N8 = LO4 ? NP - 1 : NP;  // E4M3 planes
  static_assert(AD == 1 || AD == 2, "A copied one or two steps ahead");
  constexpr int AS = AD + 1;  // A ring slots
  constexpr int NBA = NB > 0 ? NB : 1;
  constexpr int NA = CPA ? 2 * N8 + (LO4 ? 1 : 0) + 1 : 0;  // copies of A per step: 2 per E4M3 plane,
                                                             // 1 for an E2M1 one, 1 for the scales
  constexpr int NW = NB > 0 ? 3 : 0;        // copies of weights per step
  constexpr int NCOPY = NA + NW;
  constexpr int NGROUP = NP * NB;                            // MFMA groups of a step (a plane of a block)
  constexpr int NPRE = NCOPY > NGROUP ? NCOPY - NGROUP : 0;  // copies issued before them
  // copies of later steps in flight when step s starts: step s - 1's copies
  // of the weights, and of A when A is two steps ahead
  constexpr int INFLIGHT = NW + (AD == 2 ? NA : 0);
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int nsteps = (nU + 1) / 2;
  const int full = nU / 2;
  uint8_t* const aring = smem;
  uint8_t* const asc = smem + AS * kPlSlot<BM, NP, LO4>;
  uint8_t* const bring = asc + AS * kPlScale<BM> + wave * kBWavePl;

  f32x16_t acc[NBA][2];
#pragma unroll
  for (int i = 0; i < NBA; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  const int psw = pl_swz(n);
  auto copy_a = [&](int s, int p, int blk) {
    const int sc = min(s, nsteps - 1);
    const int c = (lane & 3) ^ pl_swz(16 * blk + (lane >> 2));  // lane l writes position l % 4 of row l / 4
    const int u = min(2 * sc + (c >> 1), nU - 1);
    dma16(prowp[blk] + p * pst + u * 32 + (c & 1) * 16,
          lds_addr(aring + (s % AS) * kPlSlot<BM, NP, LO4> + p * kPlPlane<BM> + (32 * wave + 16 * blk) * kPlRow));
  };
  auto copy_a4 = [&](int s) {  // the E2M1 plane: lane l writes position l % 2 of row l / 2
    const int sc = min(s, nsteps - 1);
    const int c = (lane & 1) ^ pl_swz4(lane >> 1);
    const int u = min(2 * sc + c, nU - 1);
    dma16(lrow4 + u * 16,
          lds_addr(aring + (s % AS) * kPlSlot<BM, NP, LO4> + N8 * kPlPlane<BM> + 32 * wave * (kPlRow / 2)));
  };
  auto copy_as = [&](int s) {
    const int sc = min(s, nsteps - 1);
    const int u = min(2 * sc + h, nU - 1);
    dma4(srow + (SBYTE ? (u & ~3) : 4 * u), lds_addr(asc + (s % AS) * kPlScale<BM> + wave * 256));
  };
  auto b_unit = [&](int s) { return min(2 * s + h, nU - 1); };
  auto copy_b = [&](int s, int j) {
    const int cc = b_unit(min(s, nsteps - 1));
    const uint8_t* g = btile + (int64_t)cc * 1024 + (32 * j + n) * 16;
    const uint32_t l = lds_addr(bring + (s % kBSlotsPl) * kBSlotPl + j * 1024);
    if constexpr (NT)
      dma16_nt(g, l);
    else
      dma16(g, l);
  };
  auto copy_bs = [&](int s) {
    const int cw = min(2 * min(s, nsteps - 1), nU - 1);
    dma4(btile + (int64_t)nU * 1024 + (cw / 4) * 256 + lane * 4,
         lds_addr(bring + (s % kBSlotsPl) * kBSlotPl + 2048));
  };
  // Copies of a step, always issued in this order (vm_wait counts on it):
  // with CPA, the planes' rows and the scale dwords for step s + AD; then
  // (waves with a weight tile) the 2 code halves and the scale dwords for
  // step s + 2.
  auto copy = [&](int s, int ci) {
    if (CPA && ci < 2 * N8)
      copy_a(s + AD, ci >> 1, ci & 1);
    else if (CPA && LO4 && ci == 2 * N8)
      copy_a4(s + AD);
    else if (CPA && ci == NA - 1)
      copy_as(s + AD);
    else if (ci - NA < 2)
      copy_b(s + 2, ci - NA);
    else
      copy_bs(s + 2);
  };
  auto step = [&](int s, bool tail) {
    vm_wait<INFLIGHT>();  // this wave's copies for step s have landed (those for s + 1 may not)
    __syncthreads();  // everyone's have; everyone is done with step s - 1
#pragma unroll
    for (int ci = 0; ci < NPRE; ++ci) copy(s, ci);
    if constexpr (NB > 0) {
      const uint8_t* bs = bring + (s % kBSlotsPl) * kBSlotPl;
      const uint8_t* ps = aring + (s % AS) * kPlSlot<BM, NP, LO4>;
      const uint8_t* ss = asc + (s % AS) * kPlScale<BM>;
      const int c = b_unit(s);
      const bool z = tail && h;
      i32x8_t bop[2];
      int sb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const i32x4_t w = *(const i32x4_t*)(bs + j * 1024 + lane * 16);
        const uint32_t sw = *(const uint32_t*)(bs + 2048 + (32 * j + n) * 4);
        bop[j] = z ? i32x8_t{} : i32x8_t{w[0], w[1], w[2], w[3], 0, 0, 0, 0};
        sb[j] = z ? 127 : (int)((sw >> (8 * (c & 3))) & 0xFFu);
      }
      int ci = NPRE;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const uint32_t asw = *(const uint32_t*)(ss + i * 256 + lane * 4);
#pragma unroll
        for (int p = 0; p < N8; ++p) {
          const uint8_t* pr = ps + p * kPlPlane<BM> + (i * 32 + n) * kPlRow;
          const i32x4_t a0 = *(const i32x4_t*)(pr + ((h ^ psw) * 16));
          i32x4_t a1 = *(const i32x4_t*)(pr + (((2 + h) ^ psw) * 16));
          if (tail) a1 = i32x4_t{};
          const i32x8_t aop = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          const int sa = z ? 127 : (int)((asw >> (8 * (SBYTE ? (c & 3) : p))) & 0xFFu);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop[j], acc[i][j], 0, 4, 0, sa, 0, sb[j]);
          if (ci < NCOPY) copy(s, ci++);
        }
        if constexpr (LO4) {  // E2M1 x E2M1 (cbsz 4): the lane's own unit, as B
          const i32x4_t a = *(const i32x4_t*)(ps + N8 * kPlPlane<BM> + (i * 32 + n) * (kPlRow / 2) +
                                              ((h ^ pl_swz4(n)) * 16));
          const i32x8_t aop = z ? i32x8_t{} : i32x8_t{a[0], a[1], a[2], a[3], 0, 0, 0, 0};
          const int sa = z ? 127 : (int)((asw >> (8 * N8)) & 0xFFu);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop[j], acc[i][j], 4, 4, 0, sa, 0, sb[j]);
          if (ci < NCOPY) copy(s, ci++);
        }
      }
      while (ci < NCOPY) copy(s, ci++);
    }
  };

  // the first steps' copies in the order of a step's: A(0) (and A(1) when
  // AD = 2) with the weights of steps 0 and 1
  auto copies_a = [&](int s) {
    if constexpr (CPA) {
#pragma unroll
      for (int p = 0; p < N8; ++p) {
        copy_a(s, p, 0);
        copy_a(s, p, 1);
      }
      if constexpr (LO4) copy_a4(s);
      copy_as(s);
    }
  };
  auto copies_b = [&](int s) {
    if constexpr (NB > 0) {
      copy_b(s, 0);
      copy_b(s, 1);
      copy_bs(s);
    }
  };
  copies_a(0);
  copies_b(0);
  if constexpr (AD == 2) copies_a(1);
  copies_b(1);
  for (int s = 0; s < full; ++s) step(s, false);
  if (full < nsteps) step(full, true);
  pre();         // LDS the epilogue reads, written before the barrier
  vm_wait<0>();  // no copy may land after the workgroup's LDS is released
  __syncthreads();
  if constexpr (NB > 0) epilogue(acc);
}

// gemm_main_pl with NB = the number of 32-row blocks holding the tile's rows
// (0 when the wave has no weight tile); the wave copies its A block when the
// tile has rows in it.  Tiles of BM = 32 rows have one block, copied by wave
// 0.  Each variant carries its own copy of the epilogue.
template <int BM, int NP, int AD, bool SBYTE, bool LO4, bool NT, typename Pre, typename Epilogue>
__device__ __forceinline__ void gemm_rows_pl(int rows, const uint8_t* const (&prowp)[2], int64_t pst,
                                             const uint8_t* lrow4, const uint8_t* srow, int nU,
                                             const uint8_t* __restrict__ btile, bool bok, uint8_t* smem, Pre&& pre,
                                             Epilogue&& ep) {
  const bool cpa = 32 * (threadIdx.x >> 6) < rows;
#define MOE_PL(NB, CPA) \
  gemm_main_pl<BM, NP, AD, SBYTE, LO4, NT, NB, CPA>(prowp, pst, lrow4, srow, nU, btile, smem, pre, ep)
  if constexpr (BM == 32) {
    if (!bok) {
      if (cpa)
        MOE_PL(0, true);
      else
        MOE_PL(0, false);
    } else {
      if (cpa)
        MOE_PL(1, true);
      else
        MOE_PL(1, false);
    }
  } else if (!bok) {
    if (cpa)
      MOE_PL(0, true);
    else
      MOE_PL(0, false);
  } else if (rows > 96) {
    MOE_PL(4, true);
  } else if (rows > 64) {
    if (cpa)
      MOE_PL(3, true);
    else
      MOE_PL(3, false);
  } else if (rows > 32) {
    if (cpa)
      MOE_PL(2, true);
    else
      MOE_PL(2, false);
  } else {
    if (cpa)
      MOE_PL(1, true);
    else
      MOE_PL(1, false);
  }
#undef MOE_PL
}

}  // namespace moe
