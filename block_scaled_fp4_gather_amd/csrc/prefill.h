// Host-side sizing and launch entry of the grouped (prefill) forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace moe {

constexpr int kGemmBM = 128;             // routes per m-tile of the grouped GEMMs
constexpr int kSparseRoutesPerExpert = 16;  // up to this many routes per expert on average: 32-row m-tiles
constexpr int kRouteMaxExperts = 8192;   // experts the grouping's LDS histogram holds

// Workspace of the grouped path, byte offsets (256-byte aligned).
struct PrefillWs {
  int64_t counts;      // int32 [E]   valid routes per expert
  int64_t grp_start;   // int32 [E]   first grouped row of each expert
  int64_t tile_start;  // int32 [E+1] first FC1 m-tile of each expert; [E] = total tiles
  int64_t fill;        // int32 [E]   grouped rows handed out per expert (routing)
  int64_t tile_expert; // int32 [R/32 + E] expert of each FC1 m-tile
  int64_t tile_start2; // int32 [E+1] the same for FC2's m-tiles
  int64_t tile_expert2;// int32 [R/32 + E]
  int64_t perm;        // int32 [R]   grouped row -> route index t*k + j
  int64_t rpos;        // int32 [R]   route index -> grouped row (valid routes)
  int64_t gw;          // fp32 [R]   router weight of each grouped row
  // bf16 activations a = SiLU(gate)*up per grouped row, hi = bf16(a) and
  // lo = a - hi:
  int64_t act;         // NVFP4: bf16 [R][I] hi plane, then bf16 [R][I] lo = bf16(a - hi)
                       // (16 significant bits); MXFP4: three MXFP8 planes in aq / as
  // MXFP8 activations (W4A8-MX; scale rows padded to whole dwords):
  int64_t xq;          // u8 [M][H]  x codes per token
  int64_t xs;          // u8 [M][a8_scale_stride(H)]  x scales
  int64_t aq;          // u8 [R][I]  SiLU(gate)*up codes per grouped row; MXFP4 with bf16
                       // activations: u8 [2][R][I] E4M3 (plane p at p * pst bytes) holding hi
                       // (its MXFP8 rounding, then the remainder), then u8 [R][I / 2] E2M1 lo
  int64_t as;          // u8 [R][a8_scale_stride(I)]  their scales; MXFP4 with bf16 activations:
                       // u32 [R][I / 32], byte p the scale of plane p for those 32 columns
  int64_t pst;         // bytes from one MXFP8 plane to the next (MXFP4 with bf16 activations)
  int64_t y;           // fp32 [R][H] router-weighted FC2 output per grouped row
  int64_t total;
};

// Bytes of one MXFP8 scale row of n values: n / 32 scales rounded up to
// whole dwords (the A8 GEMMs copy 4 unit scales at a time).
__host__ __device__ inline int a8_scale_stride(int n) { return (n / 32 + 3) / 4 * 4; }

// Workspace of the grouped path for `routes` routes of `tokens` tokens;
// `a8` lays out the MXFP8-activation buffers instead of the bf16 planes.
inline PrefillWs prefill_ws(const Layout& L, int64_t routes, int64_t tokens, bool a8) {
  PrefillWs w;
  w.counts = 0;
  w.grp_start = align_up(4 * (int64_t)L.E, 256);
  w.tile_start = w.grp_start + align_up(4 * (int64_t)L.E, 256);
  w.fill = w.tile_start + align_up(4 * ((int64_t)L.E + 1), 256);
  w.tile_expert = w.fill + align_up(4 * (int64_t)L.E, 256);
  w.tile_start2 = w.tile_expert + align_up(4 * ((routes + 31) / 32 + (int64_t)L.E), 256);
  w.tile_expert2 = w.tile_start2 + align_up(4 * ((int64_t)L.E + 1), 256);
  w.perm = w.tile_expert2 + align_up(4 * ((routes + 31) / 32 + (int64_t)L.E), 256);
  w.rpos = w.perm + align_up(4 * routes, 256);
  w.gw = w.rpos + align_up(4 * routes, 256);
  int64_t o = w.gw + align_up(4 * routes, 256);
  w.act = w.xq = w.xs = w.aq = w.as = o;
  w.pst = 0;
  if (a8) {
    w.xq = o;
    w.xs = w.xq + align_up(tokens * L.H, 256);
    w.aq = w.xs + align_up(tokens * a8_scale_stride(L.H), 256);
    w.as = w.aq + align_up(routes * L.I, 256);
    o = w.as + align_up(routes * a8_scale_stride(L.I), 256);
  } else if (L.fmt == kMXFP4) {
    w.pst = align_up(routes * L.I, 256);
    w.aq = o;
    w.as = w.aq + 2 * w.pst + align_up(routes * L.I / 2, 256);
    o = w.as + align_up(routes * (L.I / 32) * 4, 256);
  } else {
    w.aq = w.as = w.act + align_up(2 * routes * L.I, 256);
    o = w.act + 2 * align_up(2 * routes * L.I, 256);
  }
  w.y = o;
  w.total = w.y + align_up(4 * routes * L.H, 256);
  return w;
}

// Largest routes (M * k) the grouped path takes: grouped-row indexes stay in
// int32 and the workspace within 4 * (I + H) + 16 bytes per route (bf16
// activations; less with MXFP8 activations, plus H + H / 32 per token).
constexpr int64_t kPrefillMaxRoutes = int64_t(1) << 22;

// FC1 column blocks: 4 prepared tiles (128 gate + 128 up columns) each.
__host__ __device__ inline int fc1_blocks(const Layout& L) { return (L.nB1 + 3) / 4; }
// FC2 column blocks: 4 prepared tiles (256 output columns) each.
__host__ __device__ inline int fc2_blocks(const Layout& L) { return (L.nB2 + 3) / 4; }

// Rows of the grouped GEMMs' m-tiles for `routes` routes, each GEMM its
// own: 128, or 32 when the experts get few routes each, where most 128-row
// tiles would hold a few rows and three or four smaller workgroups per CU
// keep more weight copies in flight.  Measured on MI355X per GEMM, 32-row
// tiles stay ahead for longer in two cases: MXFP4 FC1 with bf16 activations
// (up to 64 routes per expert) and NVFP4 FC2, whose 32-row tiles take both
// activation planes in one pass (up to 128; at 114 they were 20% faster).
inline int prefill_bm1(const Layout& L, int64_t routes, bool a8) {
  const int64_t lim = !a8 && L.fmt == kMXFP4 ? 4 * kSparseRoutesPerExpert : kSparseRoutesPerExpert;
  return routes <= lim * L.E ? 32 : kGemmBM;
}
inline int prefill_bm2(const Layout& L, int64_t routes, bool a8) {
  const int64_t lim = !a8 && L.fmt == kNVFP4 ? 8 * kSparseRoutesPerExpert : kSparseRoutesPerExpert;
  return routes <= lim * L.E ? 32 : kGemmBM;
}

// Workgroups of the larger grouped GEMM grid for up to `routes` routes (a
// call with fewer routes may take 32-row tiles); the grid must stay below
// 2^31 workgroups.
inline int64_t prefill_max_workgroups(const Layout& L, int64_t routes) {
  const int64_t bm = 32;
  const int64_t mt = (routes + bm - 1) / bm + L.E;
  const int64_t nb1 = (L.I + 63) / 64, nb2 = (L.H + 127) / 128;
  return mt * (nb1 > nb2 ? nb1 : nb2) + 8;
}

// phases: 1 queues routing + FC1, 2 queues FC2 + combine (which read what
// the first part left in the workspace), 3 both; 4 queues the routing alone
// and 8 the combine alone (for timing the GEMMs apart from them).  `a8`
// selects MXFP8 activations (MXFP4 weights only): x is quantised in phase 1
// and both GEMMs run on the scaled matrix instruction.
template <typename IdT>
hipError_t launch_prefill(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                          const IdT* ids, const float* tw, uint16_t* out, uint8_t* ws,
                          const PrefillWs& W, int phases, bool a8, hipStream_t st);

// The A8 GEMM launches (x quantisation + FC1, FC2) over a grid of `grid`
// workgroups of m-tiles of `bm` rows numbered by the tables ts / te (the
// same tile grids as the bf16 GEMMs).
hipError_t launch_fc1_a8(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k, uint8_t* ws,
                         const PrefillWs& W, int bm, const int* ts, const int* te, unsigned grid, hipStream_t st);
hipError_t launch_fc2_a8(const Layout& L, const uint8_t* prep, uint8_t* ws, const PrefillWs& W, int bm,
                         const int* ts, const int* te, unsigned grid, hipStream_t st);

}  // namespace moe
