// Host-side sizing and launch entry of the decode-band forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace moe {

// The decode band keeps one route slot per lane of a wave64.
constexpr int kDecodeMaxSlots = 64;
constexpr int kDecodeMaxTokens = 16;
constexpr int kMaxWaves = 16;   // waves per FC1 workgroup
constexpr int kMaxWaves2 = 12;  // waves per FC2 workgroup (register budget)

// Workspace of the decode band: the activation a[r][n] of every route slot r
// that carries an (expert, token) pair, as two bf16 planes (hi, lo).
struct DecodeWs {
  int64_t act_hi, act_lo, total;
};

inline DecodeWs decode_ws(const Layout& L, int slots) {
  DecodeWs w;
  w.act_hi = 0;
  w.act_lo = align_up(2 * (int64_t)slots * L.I, 256);
  w.total = w.act_lo + align_up(2 * (int64_t)slots * L.I, 256);
  return w;
}

// Largest M the decode band takes for top-k routing.
inline int decode_max_tokens(int k) {
  const int m = kDecodeMaxSlots / k;
  return m < kDecodeMaxTokens ? m : kDecodeMaxTokens;
}

// FC1 K-slab width (chunks per wave): the smallest of 4, 8, 16 whose slabs
// fit in one workgroup of at most 16 waves (wider K loops over slabs).
inline int choose_slab(const Layout& L) {
  for (int cs : {4, 8})
    if ((L.nC1 + cs - 1) / cs <= kMaxWaves) return cs;
  return 16;
}

template <typename IdT>
hipError_t launch_decode(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                         const IdT* ids, const float* tw, uint16_t* out, uint8_t* ws,
                         const DecodeWs& W, int cs, int phases, hipStream_t st);

hipError_t launch_repack(const Layout& L, int dir, uint8_t* w13c, uint8_t* w13s, uint8_t* w2c,
                         uint8_t* w2s, float* g13, float* g2, uint8_t* prep, hipStream_t st);

hipError_t launch_export(const Layout& L, int e, int which, const uint8_t* prep, float* out,
                         hipStream_t st);

}  // namespace moe
