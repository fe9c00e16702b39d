// Grouped GEMMs of the W4A8-MX variant: MXFP8 activation rows times MXFP4
// weights on the CDNA4 scaled matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4 (A: E4M3, B: E2M1, one E8M0 scale per 32
// K values of each row and column, fp32 accumulation): 128-row m-tiles in the
// loop below, 32-row ones in the plane loop with one plane.  The FP4 weights and their UE8M0 bytes enter the
// instruction as stored, with no decode (b12x PR #22, Measured table: the A8
// path keeps its prefill advantage; the dynamic path quantises activations to
// MXFP8).
//
//   fc1_gemm_a8  x rows (MXFP8, quantised once per token) gathered by
//                grouped row, the activation f(gate, up) in fp32 (relu2:
//                both halves as outputs), quantised to MXFP8 in blocks of 32
//                along I (the 32 columns of one wave's prepared tile are one
//                block) -> act codes and scales;
//   fc2_gemm_a8  act rows times W2, times the grouped row's router weight ->
//                the same fp32 rows that the combine sums.
#include <hip/hip_runtime.h>

#include "act.h"
#include "gemm_planes.h"
#include "gemm_util.h"
#include "layout.h"
#include "mxfp8.h"
#include "prefill.h"

namespace moe {

// LDS of an A8 workgroup: A ring of 2 slots x 128 rows x 128 bytes (128 K
// values of FP8, the 16-byte chunk c of row r at position c ^ swz(r)); A
// scale ring of 2 slots x 4 waves x 256 bytes (rows 32w..32w+31 of the tile,
// one dword of 4 unit scales per row; the upper 128 bytes are spare); weight
// ring of 2 slots x 4 waves x (4 x 1 KiB codes + 256 B of scale dwords, one
// per weight row, + 256 B spare).
constexpr int kStepK8 = 128;                 // K values per main-loop step (4 units)
constexpr int kARow8 = kStepK8;              // bytes of one A row of a step
constexpr int kAPlane8 = kGemmBM * kARow8;   // 16 KiB
constexpr int kASlot8 = 4 * 256;
constexpr int kBWave8 = 4 * 1024 + 2 * 256;
constexpr int kBSlot8 = 4 * kBWave8;
constexpr int kGemmLds8 = 2 * kAPlane8 + 2 * kASlot8 + 2 * kBSlot8;

__device__ __forceinline__ i32x4_t lds16(const uint8_t* p) { return *(const i32x4_t*)p; }

// Byte b of a dword as an E8M0 scale operand (the instruction reads the low
// byte with op_sel 0).
__device__ __forceinline__ int scale_byte(uint32_t w, int b) { return (int)((w >> (8 * b)) & 0xFFu); }

// Main loop for one 128-row x 256-column output tile of the A8 GEMMs,
// followed by `epilogue(acc)` (32-row tiles take the plane loop, whose steps
// of 64 K values suit their single row block; with four row blocks this
// loop's steps of 128 share each barrier among twice the MFMAs, measured 12%
// faster on full tiles).  K runs over nU units of 32 values in steps
// of 4 units; MFMA t (0, 1) of a step takes units 2t and 2t + 1.
//
// Wave w owns the 64 columns of one prepared weight tile (`btile`, nU
// chunks) and the first 32 * NB rows (NB = 1..4; 0 for a wave past the last
// weight tile, which only helps stage A).  Every copy of step s + 1 is
// issued during step s: A rows (wave w copies rows 32w..32w+31 of the tile,
// 8 rows per copy, from `rowp[blk]`), their scale dwords (from `srow`, this
// lane's row 32w + lane % 32), and the wave's weights, which lane (n, h)
// copies for the units it multiplies (unit 4s + 2t + h of weight rows n and
// 32 + n), with one copy of the scale dwords of all 64 rows.  Copies past
// the last unit are clamped to it; in a last step with fewer than 4 units
// the absent units' operands are zeroed and their scales set to 1 when read.
template <int NB, typename Epilogue>
__device__ __forceinline__ void gemm_main_a8(const uint8_t* const (&rowp)[4], const uint8_t* srow, int nU,
                                             const uint8_t* __restrict__ btile, uint8_t* smem,
                                             Epilogue&& epilogue) {
  constexpr int NBA = NB > 0 ? NB : 1;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int nsteps = (nU + 3) / 4;
  const int full = nU / 4;
  uint8_t* const aring = smem;
  uint8_t* const sring = smem + 2 * kAPlane8;
  uint8_t* const bring = smem + 2 * kAPlane8 + 2 * kASlot8 + wave * kBWave8;

  f32x16_t acc[NBA][2];
#pragma unroll
  for (int i = 0; i < NBA; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  const int cp_lo = (lane & 7) ^ (lane >> 3);
  const int swz = a_swz(n);
  auto copy_a = [&](int s, int blk) {
    const int sc = min(s, nsteps - 1);
    const int c = cp_lo ^ (blk & 1);
    const int u = min(4 * sc + (c >> 1), nU - 1);
    dma16(rowp[blk] + u * 32 + (c & 1) * 16,
          lds_addr(aring + (s & 1) * kAPlane8 + (32 * wave + 8 * blk) * kARow8));
  };
  auto copy_as = [&](int s) {
    dma4(srow + 4 * min(s, nsteps - 1), lds_addr(sring + (s & 1) * kASlot8 + wave * 256));
  };
  auto copy_b = [&](int s, int q) {  // q = 2t + j
    const int sc = min(s, nsteps - 1);
    const int tt = q >> 1, j = q & 1;
    const int u = min(4 * sc + 2 * tt + h, nU - 1);
    dma16(btile + (int64_t)u * 1024 + (32 * j + n) * 16, lds_addr(bring + (s & 1) * kBSlot8 + q * 1024));
  };
  // the scale dwords of the step's 4 units for all 64 weight rows (lane l: row l)
  auto copy_bs = [&](int s) {
    const int sc = min(s, nsteps - 1);
    dma4(btile + (int64_t)nU * 1024 + sc * 256 + lane * 4, lds_addr(bring + (s & 1) * kBSlot8 + 4096));
  };
  // copies of one step, in issue order: 4 A row blocks, the A scales, then
  // (waves with a weight tile) 4 weight unit sets and the weight scales
  constexpr int NCOPY = NB > 0 ? 10 : 5;
  auto copy = [&](int s, int ci) {
    if (ci < 4)
      copy_a(s, ci);
    else if (ci == 4)
      copy_as(s);
    else if (ci < 9)
      copy_b(s, ci - 5);
    else
      copy_bs(s);
  };

  auto step = [&](int s, int rem) {  // rem: units of this step (4 unless the last)
    vm_wait<0>();     // this wave's copies of step s have landed
    __syncthreads();  // everyone's have; everyone is done with step s - 1
    if constexpr (NB == 0) {
#pragma unroll
      for (int ci = 0; ci < NCOPY; ++ci) copy(s + 1, ci);
    } else {
      const uint8_t* bs = bring + (s & 1) * kBSlot8;
      const uint8_t* as = aring + (s & 1) * kAPlane8;
      const uint8_t* ss = sring + (s & 1) * kASlot8;
      uint32_t bsw[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) bsw[j] = *(const uint32_t*)(bs + 4096 + (32 * j + n) * 4);
      int ci = 0;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bool blk_ok[2] = {2 * tt < rem, 2 * tt + 1 < rem};
        const bool mine_ok = 2 * tt + h < rem;
        i32x8_t bop[2];
        int sb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const i32x4_t w = lds16(bs + (2 * tt + j) * 1024 + lane * 16);
          bop[j] = i32x8_t{w[0], w[1], w[2], w[3], 0, 0, 0, 0};
          sb[j] = scale_byte(bsw[j], 2 * tt + h);
          if (!mine_ok) {
            bop[j] = i32x8_t{};
            sb[j] = 127;
          }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const uint8_t* ar = as + (i * 32 + n) * kARow8;
          i32x4_t a0 = lds16(ar + (((4 * tt + h) ^ swz) * 16));
          i32x4_t a1 = lds16(ar + (((4 * tt + 2 + h) ^ swz) * 16));
          if (!blk_ok[0]) a0 = i32x4_t{};
          if (!blk_ok[1]) a1 = i32x4_t{};
          const i32x8_t aop = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          const uint32_t asw = *(const uint32_t*)(ss + i * 256 + n * 4);
          const int sa = mine_ok ? scale_byte(asw, 2 * tt + h) : 127;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop[j], acc[i][j], 0, 4, 0, sa, 0,
                                                                        sb[j]);
          // spread the next step's copies between the MFMA pairs
          if (ci < NCOPY) copy(s + 1, ci++);
          if (ci < NCOPY && (i & 1)) copy(s + 1, ci++);
        }
      }
      while (ci < NCOPY) copy(s + 1, ci++);
    }
  };

#pragma unroll
  for (int ci = 0; ci < NCOPY; ++ci) copy(0, ci);
  for (int s = 0; s < full; ++s) step(s, 4);
  if (full < nsteps) step(full, nU - 4 * full);
  vm_wait<0>();  // the clamped copies issued in the last step have landed
  __syncthreads();
  if constexpr (NB > 0) epilogue(acc);
}

template <typename Epilogue>
__device__ __forceinline__ void gemm_rows_a8(int rows, const uint8_t* const (&rowp)[4], const uint8_t* srow,
                                             int nU, const uint8_t* __restrict__ btile, bool bok, uint8_t* smem,
                                             Epilogue&& ep) {
  if (!bok)
    gemm_main_a8<0>(rowp, srow, nU, btile, smem, ep);
  else if (rows > 96)
    gemm_main_a8<4>(rowp, srow, nU, btile, smem, ep);
  else if (rows > 64)
    gemm_main_a8<3>(rowp, srow, nU, btile, smem, ep);
  else if (rows > 32)
    gemm_main_a8<2>(rowp, srow, nU, btile, smem, ep);
  else
    gemm_main_a8<1>(rowp, srow, nU, btile, smem, ep);
}

// Occupancy (waves per SIMD): two 128-row workgroups per CU (the
// accumulators of four row blocks), four of 32 rows.
template <int BM>
constexpr int kA8Waves = BM == 32 ? 4 : 2;

template <int BM>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kA8Waves<BM>)))
    fc1_gemm_a8(const uint8_t* __restrict__ prep, const Layout L, const uint8_t* __restrict__ xq,
                const uint8_t* __restrict__ xs, int xss, int k, const int* __restrict__ counts,
                const int* __restrict__ grp_start, const int* __restrict__ tile_start,
                const int* __restrict__ tile_expert, const int* __restrict__ perm, uint8_t* __restrict__ aq,
                uint8_t* __restrict__ as, int ass) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[BM == 32 ? kPlLds<32, 1, 1, false> : kGemmLds8];
  const GroupTile id = group_tile(fc1_blocks(L), tile_start, tile_expert, L.E);
  if (!id.ok) return;
  const int e = id.e;
  const int m0 = (id.gm - tile_start[e]) * BM;
  const int rows = min(BM, counts[e] - m0);
  const int gs = grp_start[e] + m0;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int b = 4 * id.nb + wave;  // prepared FC1 tile: gate columns 32b.. and the matching up columns
  const bool bok = b < L.nB1;
  // the scale row of row 32 wave + lane % 32 of the tile (grouped rows past
  // the tile repeat its last row), a token's
  const uint8_t* srow = xs + (int64_t)(perm[gs + min(32 * wave + (lane & 31), rows - 1)] / k) * xss;
  // Epilogue, per 32-row block: a = f(gate, up) in fp32 goes to this wave's
  // part of the (now idle) A ring as 32 rows x 32 columns (row stride 144 B),
  // then lane l takes row l / 2, columns 16 (l % 2) .. + 15: the block
  // maximum is its own 16 values and its neighbour's, and its 16 codes leave
  // in one 16-byte store.  A non-gated activation (relu2) makes two such
  // blocks per row block, columns 32b.. from the first accumulator and
  // Ip + 32b.. from the second.
  auto epilogue = [&](auto& acc) __attribute__((always_inline)) {
    constexpr int NB = sizeof(acc) / sizeof(acc[0]);
    constexpr int kStride = 36;  // dwords per staged row
    float* st = (float*)(smem + wave * 32 * kStride * 4);
    const int n = lane & 31;
    const int rr = lane >> 1, half = lane & 1;
    with_act_kind(L.act.kind, [&](auto kind) __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
#pragma unroll
      for (int jj = 0; jj < (K == kActRelu2 ? 2 : 1); ++jj) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          st[acc_row(r, lane) * kStride + n] =
              K == kActRelu2 ? act_of<K>(L.act, acc[i][jj][r], 0.0f) : act_of<K>(L.act, acc[i][0][r], acc[i][1][r]);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging stores are done
        __builtin_amdgcn_wave_barrier();
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f = *(const float4*)(st + rr * kStride + 16 * half + 4 * q);
          v[4 * q] = f.x;
          v[4 * q + 1] = f.y;
          v[4 * q + 2] = f.z;
          v[4 * q + 3] = f.w;
        }
        uint32_t m = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) m = max(m, __float_as_uint(v[q]) & 0x7FFFFFFFu);
        m = max(m, (uint32_t)__shfl_xor((int)m, 1));
        const uint32_t sb = mx_scale_byte(m);
        uint32_t w[4] = {0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};
        if (sb != 255u) {
          const float inv = mx_inv_scale(sb);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            w[q] = e4m3_code(v[4 * q] * inv) | (e4m3_code(v[4 * q + 1] * inv) << 8) |
                   (e4m3_code(v[4 * q + 2] * inv) << 16) | (e4m3_code(v[4 * q + 3] * inv) << 24);
        }
        const int row = i * 32 + rr;
        const int col0 = (jj ? L.Ip : 0) + 32 * b;
        if (row < rows) {
          *(uint4*)(aq + (int64_t)(gs + row) * L.I + col0 + 16 * half) = make_uint4(w[0], w[1], w[2], w[3]);
          if (half == 0) as[(int64_t)(gs + row) * ass + col0 / 32] = (uint8_t)sb;
        }
        __builtin_amdgcn_wave_barrier();  // the next block's stores come after these reads
        __builtin_amdgcn_s_waitcnt(0xC07F);
      }
    }
    });
  };
  const uint8_t* btile = prep + fc1_tile_offset(L, e, bok ? b : 0);
  if constexpr (BM == 32) {
    // x rows this lane copies: rows 32 wave + 16 blk + lane / 4 of the tile
    const uint8_t* prowp[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
      prowp[blk] = xq + (int64_t)(perm[gs + min(32 * wave + 16 * blk + (lane >> 2), rows - 1)] / k) * L.H;
    gemm_rows_pl<BM, 1, 1, true, false, true>(rows, prowp, 0, nullptr, srow, L.nC1, btile, bok, smem, [] {}, epilogue);
  } else {
    // x rows this lane copies: rows 32 wave + 8 blk + lane / 8 of the tile
    const uint8_t* rowp[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
      rowp[blk] = xq + (int64_t)(perm[gs + min(32 * wave + 8 * blk + (lane >> 3), rows - 1)] / k) * L.H;
    gemm_rows_a8(rows, rowp, srow, L.nC1, btile, bok, smem, epilogue);
  }
}

template <int BM>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kA8Waves<BM>)))
    fc2_gemm_a8(const uint8_t* __restrict__ prep, const Layout L, const float* __restrict__ gw,
                const int* __restrict__ counts, const int* __restrict__ grp_start,
                const int* __restrict__ tile_start, const int* __restrict__ tile_expert,
                const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as, int ass, float* __restrict__ y) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[BM == 32 ? kPlLds<32, 1, 2, false> : kGemmLds8];
  __shared__ float wrow[BM];
  const GroupTile id = group_tile(fc2_blocks(L), tile_start, tile_expert, L.E);
  if (!id.ok) return;
  const int e = id.e;
  const int m0 = (id.gm - tile_start[e]) * BM;
  const int rows = min(BM, counts[e] - m0);
  const int gs = grp_start[e] + m0;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int hb = 4 * id.nb + wave;  // prepared FC2 tile: output columns 64hb..64hb+63
  const bool bok = hb < L.nB2;
  // the router weights of the tile's rows, loaded now and put in LDS after
  // the main loop (no copy waits for them)
  const float wv = t < rows ? gw[gs + t] : 0.0f;
  auto pre = [&] {
    if (t < BM) wrow[t] = wv;
  };
  // the scale row of row 32 wave + lane % 32 of the tile
  const uint8_t* srow = as + (int64_t)(gs + min(32 * wave + (lane & 31), rows - 1)) * ass;
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
          y[(int64_t)(gs + row) * L.H + n] = acc[i][j][r] * wrow[row];
        }
      }
    }
  };
  const uint8_t* btile = prep + fc2_tile_offset(L, e, bok ? hb : 0);
  if constexpr (BM == 32) {
    // act rows this lane copies: rows 32 wave + 16 blk + lane / 4 of the tile,
    // two steps ahead (FC1, whose x rows are gathered, copies them one step
    // ahead: measured 5% faster there, while FC2 was 8% faster two ahead)
    const uint8_t* prowp[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
      prowp[blk] = aq + (int64_t)(gs + min(32 * wave + 16 * blk + (lane >> 2), rows - 1)) * L.I;
    gemm_rows_pl<BM, 1, 2, true, false, true>(rows, prowp, 0, nullptr, srow, L.nC2, btile, bok, smem, pre, epilogue);
  } else {
    // act rows this lane copies: rows 32 wave + 8 blk + lane / 8 of the tile;
    // the router weights go to LDS before the main loop, whose barriers
    // order them before the epilogue
    const uint8_t* rowp[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
      rowp[blk] = aq + (int64_t)(gs + min(32 * wave + 8 * blk + (lane >> 3), rows - 1)) * L.I;
    pre();
    gemm_rows_a8(rows, rowp, srow, L.nC2, btile, bok, smem, epilogue);
  }
}

hipError_t launch_fc1_a8(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k, uint8_t* ws,
                         const PrefillWs& W, int bm, const int* ts, const int* te, unsigned grid, hipStream_t st) {
  uint8_t* xq = ws + W.xq;
  uint8_t* xs = ws + W.xs;
  hipError_t err = launch_mxfp8_quantize(x, M, L.H, xq, xs, a8_scale_stride(L.H), st);
  if (err != hipSuccess) return err;
#define MOE_FC1A8(BM)                                                                                           \
  hipLaunchKernelGGL(fc1_gemm_a8<BM>, dim3(grid), dim3(256), 0, st, prep, L, (const uint8_t*)xq,               \
                     (const uint8_t*)xs, a8_scale_stride(L.H), k, (const int*)(ws + W.counts),                  \
                     (const int*)(ws + W.grp_start), ts, te, (const int*)(ws + W.perm), ws + W.aq, ws + W.as,   \
                     a8_scale_stride(L.I))
  if (bm == 32)
    MOE_FC1A8(32);
  else
    MOE_FC1A8(kGemmBM);
#undef MOE_FC1A8
  return hipGetLastError();
}

hipError_t launch_fc2_a8(const Layout& L, const uint8_t* prep, uint8_t* ws, const PrefillWs& W, int bm,
                         const int* ts, const int* te, unsigned grid, hipStream_t st) {
#define MOE_FC2A8(BM)                                                                                           \
  hipLaunchKernelGGL(fc2_gemm_a8<BM>, dim3(grid), dim3(256), 0, st, prep, L, (const float*)(ws + W.gw),        \
                     (const int*)(ws + W.counts), (const int*)(ws + W.grp_start), ts, te,                        \
                     (const uint8_t*)(ws + W.aq), (const uint8_t*)(ws + W.as),                                   \
                     a8_scale_stride(L.I), (float*)(ws + W.y))
  if (bm == 32)
    MOE_FC2A8(32);
  else
    MOE_FC2A8(kGemmBM);
#undef MOE_FC2A8
  return hipGetLastError();
}

}  // namespace moe
