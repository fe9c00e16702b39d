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
// Activations of all route slots are staged in FC2's LDS up to this size,
// within the 64 KiB a workgroup may allocate without opting in to more.
constexpr int64_t kStageActBytes = 40 * 1024;
constexpr int64_t kMaxLdsBytes = 64 * 1024;

// Waves per FC2 workgroup: 16-chunk lanes need more than the 128 VGPRs a
// 16-wave workgroup leaves each wave.
constexpr int fc2_max_waves(int kl) { return kl >= 16 ? 12 : 16; }

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

// Largest M one decode launch pair takes for top-k routing.
inline int decode_max_tokens(int k) {
  const int m = kDecodeMaxSlots / k;
  return m < kDecodeMaxTokens ? m : kDecodeMaxTokens;
}

// Launch shape of the decode kernels (see moe_fp4_tuning).
struct DecodeShape {
  int kl1;  // FC1 chunks per wave: 4, 8, 16
  int r1;   // FC1 rows per workgroup: 16, 32
  int r2;   // FC2 rows per workgroup: 8, 16, 32
};

// FC2 chunk lanes: 4 up to 4 chunks of I, 8 up to 16 (two groups of 8
// chunks, loaded together), else 16 (longer I loops).  With 8 lanes a load
// instruction reads 8 consecutive rows of each chunk, whole 128-byte lines;
// 16 lanes read 4 rows (half lines).
inline int fc2_chunk_lanes(const Layout& L) { return L.nC2 <= 4 ? 4 : (L.nC2 <= 16 ? 8 : 16); }

// Chunk groups an FC2 lane loads at once: 2 for 8 lanes over 9..16 chunks.
inline int fc2_chunk_groups(const Layout& L) { return fc2_chunk_lanes(L) == 8 && L.nC2 > 8 ? 2 : 1; }

// Decode kernels with compressed scales keep each row's base byte and offsets
// in registers: FC1 with 16 chunk lanes and 32 rows (8 rows per lane), and
// FC2 with 32 rows over two chunk groups (8 units per lane), would spill,
// so those shapes are not taken for layouts with compressed scales.
constexpr bool csf_shape_ok(int fc2_kl, int r2, int fc2_ci) { return !(fc2_ci == 2 && r2 * fc2_kl / 64 * fc2_ci > 4); }

inline bool valid_shape(const Layout& L, const DecodeShape& s) {
  if (L.csf && s.kl1 == 16 && s.r1 == 32) return false;
  if (L.csf && s.r2 != 0 && !csf_shape_ok(fc2_chunk_lanes(L), s.r2, fc2_chunk_groups(L))) return false;
  if (s.kl1 != 0 && s.kl1 != 4 && s.kl1 != 8 && s.kl1 != 16) return false;
  if (s.r1 != 0 && s.r1 != 16 && s.r1 != 32) return false;
  if (s.r2 != 0 && s.r2 != 8 && s.r2 != 16 && s.r2 != 32) return false;
  if (s.r2 != 0 && s.r2 * fc2_chunk_lanes(L) < 64) return false;  // a lane needs a row
  return true;
}

// Built-in choices for fields left at 0, from sweeps on MI355X over the
// E512/H2560/I320 NVFP4 (M = 1), E288/H4096/I512 NVFP4 (M = 5) and
// E256/H7168/I256 MXFP4 (M = 1, 2, 4) decode shapes:
//  - FC1 takes 4 chunks per wave (2 rows per lane, waves loop over more
//    chunk groups) for K up to 128 chunks and from 16 route slots on, where
//    it was 13-26% faster than 8 (21% on E288/H4096 at M = 1); with longer
//    K (4 chunk groups per wave) and fewer slots 8 is faster;
//  - FC2 takes 32-row blocks when its lanes cover I in one group of at most
//    8 chunks (I <= 256), 24-27% faster than 16 rows from M = 2 on; with two
//    groups (I up to 512) or 16 chunk lanes, 16 rows (32 rows were 26-36%
//    slower there, 8 rows 14-60%).
inline DecodeShape resolve_shape(const Layout& L, int slots, DecodeShape s) {
  if (s.kl1 == 0) s.kl1 = (L.nC1 <= 128 || slots >= 16) ? 4 : 8;
  if (s.r1 == 0) s.r1 = (int64_t)slots * L.nB1 * 2 >= 160 ? 32 : 16;
  if (s.r2 == 0) s.r2 = fc2_chunk_lanes(L) <= 8 && fc2_chunk_groups(L) == 1 ? 32 : 16;
  return s;
}

// Dynamic LDS of an FC1 workgroup: the token's H activations (bf16) and the
// per-wave partial sums of mc tokens x 16 waves x r1 rows (fp32).
inline int64_t fc1_lds_bytes(const Layout& L, int mc, int r1) {
  return 2 * align_up(L.H, 64) + (int64_t)mc * kMaxWaves * r1 * 4;
}

template <typename IdT>
hipError_t launch_decode(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                         const IdT* ids, const float* tw, uint16_t* out, uint8_t* ws,
                         const DecodeWs& W, const DecodeShape& shape, int phases, hipStream_t st);

hipError_t launch_repack(const Layout& L, int dir, uint8_t* w13c, uint8_t* w13s, uint8_t* w2c,
                         uint8_t* w2s, float* g13, float* g2, uint8_t* prep, hipStream_t st);

hipError_t launch_export(const Layout& L, int e, int which, const uint8_t* prep, float* out,
                         hipStream_t st);

}  // namespace moe
