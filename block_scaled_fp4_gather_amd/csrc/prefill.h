// Host-side sizing and launch entry of the grouped (prefill) forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace moe {

constexpr int kGemmBM = 128;             // routes per m-tile of the grouped GEMMs
constexpr int kRouteMaxExperts = 8192;   // experts the grouping's LDS histogram holds

// Workspace of the grouped path, byte offsets (256-byte aligned).
struct PrefillWs {
  int64_t counts;      // int32 [E]   valid routes per expert
  int64_t grp_start;   // int32 [E]   first grouped row of each expert
  int64_t tile_start;  // int32 [E+1] first m-tile of each expert; [E] = total tiles
  int64_t perm;        // int32 [R]   grouped row -> route index t*k + j
  int64_t rpos;        // int32 [R]   route index -> grouped row (valid routes)
  int64_t act;         // bf16 [2][R][I] SiLU(gate)*up per grouped row: hi plane, then
                       // lo plane (hi = bf16(a), lo = bf16(a - hi): 16 significant bits)
  int64_t y;           // fp32 [R][H] router-weighted FC2 output per grouped row
  int64_t total;
};

inline PrefillWs prefill_ws(const Layout& L, int64_t routes) {
  PrefillWs w;
  w.counts = 0;
  w.grp_start = align_up(4 * (int64_t)L.E, 256);
  w.tile_start = w.grp_start + align_up(4 * (int64_t)L.E, 256);
  w.perm = w.tile_start + align_up(4 * ((int64_t)L.E + 1), 256);
  w.rpos = w.perm + align_up(4 * routes, 256);
  w.act = w.rpos + align_up(4 * routes, 256);
  w.y = w.act + 2 * align_up(2 * routes * L.I, 256);
  w.total = w.y + align_up(4 * routes * L.H, 256);
  return w;
}

// Largest routes (M * k) the grouped path takes: grouped-row indexes stay in
// int32 and the workspace within 4 * (I + H) bytes per route.
constexpr int64_t kPrefillMaxRoutes = int64_t(1) << 22;

// Workgroups of the larger grouped GEMM grid for `routes` routes; the grid
// must stay below 2^31 workgroups.
inline int64_t prefill_max_workgroups(const Layout& L, int64_t routes) {
  const int64_t mt = (routes + kGemmBM - 1) / kGemmBM + L.E;
  const int64_t nb1 = (L.I + 63) / 64, nb2 = (L.H + 127) / 128;
  return mt * (nb1 > nb2 ? nb1 : nb2) + 8;
}

// phases: 1 queues routing + FC1, 2 queues FC2 + combine (which read what
// the first part left in the workspace), 3 both; 4 queues the routing alone
// and 8 the combine alone (for timing the GEMMs apart from them).
template <typename IdT>
hipError_t launch_prefill(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                          const IdT* ids, const float* tw, uint16_t* out, uint8_t* ws,
                          const PrefillWs& W, int phases, hipStream_t st);

}  // namespace moe
