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

// Forms of the decode band.  Two-pass: FC1 writes the activation, FC2 reads
// it.  Split: the FC1 launch also streams the W2 columns that belong to each
// FC1 tile and writes FC2 partial sums over them; a second, weight-free
// launch sums the partials per token.
enum { kFormAuto = 0, kFormTwoPass = 1, kFormSplit = 2 };

// W2 half-units a lane of the split kernel holds in registers (FC2 tiles
// per wave times the chunks of one FC1 tile: 1 gated, 2 for relu2's halves).
constexpr int kSplitMaxUnits = 16;
// Waves of a split-kernel workgroup (as an FC1 workgroup).
constexpr int kSplitMaxWaves = 16;
// Largest partial-sum buffer the workspace is sized for.
constexpr int64_t kSplitMaxPartBytes = 64ll << 20;

// Waves of an FC1 workgroup with KL chunks per wave.
inline int fc1_waves(const Layout& L, int kl) {
  const int groups = (L.nC1 + kl - 1) / kl;
  return groups < kMaxWaves ? groups : kMaxWaves;
}

inline int split_chunks(const Layout& L) { return L.Ip == L.I ? 1 : 2; }

// Partial sums: one fp32 row of H per route slot and 16-column block of the
// intermediate (two per FC1 tile).
inline int64_t split_part_bytes(const Layout& L, int slots) {
  return (int64_t)slots * 2 * L.nB1 * L.H * 4;
}

inline size_t split_lds(const Layout& L, int M, int waves) {
  return 2 * (size_t)align_up(L.H, 64) + (size_t)M * waves * 32 * 4 + (size_t)M * 32 * 4;
}

// FC2 tiles per wave of the split kernel (its register arrays hold 4 or 8).
inline int split_tiles_per_wave(const Layout& L, int kl) {
  const int w = fc1_waves(L, kl);
  return (L.nB2 + w - 1) / w <= 4 ? 4 : 8;
}

// Whether the split kernel can run M tokens with KL chunks per wave.
inline bool split_fits(const Layout& L, int M, int kl) {
  if (kl != 4 && kl != 8) return false;
  const int w = fc1_waves(L, kl);
  if (w > kSplitMaxWaves) return false;
  const int nt = (L.nB2 + w - 1) / w;
  if (nt > 8 || split_tiles_per_wave(L, kl) * split_chunks(L) > kSplitMaxUnits) return false;
  return split_lds(L, M, w) <= (size_t)kMaxLdsBytes;
}

// FC1 chunks per wave when the caller leaves it to the library.
inline int default_kl1(const Layout& L) { return L.nC1 <= 8 ? 4 : 8; }

// Workspace of the decode band: the activation a[r][n] of every route slot r
// that carries an (expert, token) pair, as two bf16 planes (hi, lo), for
// the two-pass form; the FC2 partial sums part[r][q][h] (fp32, 16-column
// block q of the intermediate) for the split form, when that form fits the
// shape.
struct DecodeWs {
  int64_t act_hi, act_lo, part, total;
  bool split;  // part is sized
};

inline DecodeWs decode_ws(const Layout& L, int slots) {
  DecodeWs w;
  w.act_hi = 0;
  w.act_lo = align_up(2 * (int64_t)slots * L.I, 256);
  w.part = w.act_lo + align_up(2 * (int64_t)slots * L.I, 256);
  w.split = split_part_bytes(L, slots) <= kSplitMaxPartBytes && split_fits(L, 1, default_kl1(L));
  w.total = w.part + (w.split ? align_up(split_part_bytes(L, slots), 256) : 0);
  return w;
}

// Largest M the decode band takes for top-k routing.
inline int decode_max_tokens(int k) {
  const int m = kDecodeMaxSlots / k;
  return m < kDecodeMaxTokens ? m : kDecodeMaxTokens;
}

// Launch shape of the decode kernels (see moe_fp4_tuning).
struct DecodeShape {
  int kl1;   // FC1 chunks per wave: 4, 8, 16
  int r1;    // FC1 rows per workgroup: 16, 32 (two-pass form)
  int r2;    // FC2 rows per workgroup: 8, 16, 32 (two-pass form)
  int form;  // kFormAuto, kFormTwoPass, kFormSplit
};

// FC2 chunk lanes: the smallest of 4, 8, 16 that covers I (longer I loops).
inline int fc2_chunk_lanes(const Layout& L) { return L.nC2 <= 4 ? 4 : (L.nC2 <= 8 ? 8 : 16); }

inline bool valid_shape(const Layout& L, const DecodeShape& s) {
  if (s.kl1 != 0 && s.kl1 != 4 && s.kl1 != 8 && s.kl1 != 16) return false;
  if (s.r1 != 0 && s.r1 != 16 && s.r1 != 32) return false;
  if (s.r2 != 0 && s.r2 != 8 && s.r2 != 16 && s.r2 != 32) return false;
  if (s.r2 != 0 && s.r2 * fc2_chunk_lanes(L) < 64) return false;  // a lane needs a row
  if (s.form != kFormAuto && s.form != kFormTwoPass && s.form != kFormSplit) return false;
  return true;
}

// Whether the split form can run this call.
inline bool split_usable(const Layout& L, const DecodeWs& W, int M, int kl) {
  return W.split && split_fits(L, M, kl);
}

// Built-in choices for fields left at 0 (from sweeps on MI355X over the
// E512/H2560/I320 NVFP4 and E256/H7168/I256 MXFP4 decode shapes).  Returns
// false when the split form was asked for and cannot run.
inline bool resolve_shape(const Layout& L, const DecodeWs& W, int M, int slots, DecodeShape* s) {
  if (s->kl1 == 0) s->kl1 = default_kl1(L);  // longer K: waves loop over chunk groups
  if (s->r1 == 0) s->r1 = (int64_t)slots * L.nB1 * 2 >= 160 ? 32 : 16;
  if (s->r2 == 0) s->r2 = fc2_chunk_lanes(L) == 4 ? 32 : 16;
  const bool split_ok = split_usable(L, W, M, s->kl1);
  if (s->form == kFormAuto) s->form = split_ok ? kFormSplit : kFormTwoPass;
  return s->form != kFormSplit || split_ok;
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
