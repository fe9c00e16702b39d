// Resident (prepared) weight layout for the gfx950 kernels.
//
// The logical tensors hold, per expert, W13 [2I][H] and W2 [H][I] as E2M1
// nibbles (two per byte, low nibble first) with one scale byte per G = 32
// (MXFP4, UE8M0) or G = 16 (NVFP4, E4M3) consecutive K elements.  Preparation
// keeps every byte and only moves it (b12x PR #459, "Reduce NVFP4-CSF scale
// reconstruction overhead": native nibbles and scale bytes, no requantisation,
// resident offsets reordered for contiguous decoding).
//
// Unit: 32 consecutive K elements of one row = 16 code bytes, plus 4 bytes of
// scales for every 4 (MXFP4) or 2 (NVFP4) units.
//
// A tile is 64 rows, one per lane of a wave64.  Inside a tile:
//   codes : [chunk c][lane l][16 B]   -> one wave load of chunk c reads 1 KiB
//                                        contiguous, lane l gets row l's unit
//   scales: [group q][lane l][4 B]    -> bytes 4q..4q+3 of row l's scale row
// FC1 tile b of an expert holds gate rows 32b..32b+31 in lanes 0..31 and the
// matching up rows I+32b..I+32b+31 in lanes 32..63, so SiLU(gate)*up pairs
// lane l with lane l+32.  With a non-gated activation (relu2) W13 has I rows,
// and tile b holds rows 32b.. and I/2+32b.. of it the same way (Ip = I/2
// row pairs instead of I), two independent outputs per lane pair.  FC2 tile hb holds rows 64hb..64hb+63 of W2 (rows
// past H are zero padding).  Padding bytes are zero and are never read as
// weights of a real row.
//
// Buffer: [NVFP4 globals g13[E], g2[E], padded to 256 B] then E experts, each
// [FC1 tiles][FC2 tiles], expert stride a multiple of 256 B.
//
// Compressed scales (b12x PR #459, "Reduce NVFP4-CSF scale reconstruction
// overhead", commit messages: one-bit MXFP4 and four-bit NVFP4 offsets from
// a row base byte).  With the compressed scale format every tile also holds,
// after its plain scale words, a CSF block of its 64 rows:
//   [group g][lane l][4 B]   one word per row and group of chunks: byte 0 the
//                            row's base byte (its smallest scale byte, or 255:
//                            the row is an exception and its plain scale words
//                            hold its scales), then the offsets of the group's
//                            chunks: MXFP4 24 chunks, bit 8+j the offset (0/1)
//                            of chunk 24g+j; NVFP4 3 chunks, byte 1+j those of
//                            chunk 3g+j (low nibble: its first 16 elements,
//                            high nibble: the second 16)
// so that a chunk's scale byte is base + offset, and a lane reads one word per
// row and chunk, as with the plain words.  The decode kernels read the CSF
// block; the grouped GEMMs and the inverse preparation read the plain scale
// words, which stay in place.
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifndef MOE_HD
#define MOE_HD __host__ __device__
#endif

namespace moe {

enum { kMXFP4 = 1, kNVFP4 = 2 };

// Gated activation applied to (gate, up) in the FC1 epilogues.
enum { kActSilu = 0, kActGeluTanh = 1, kActSwigluOai = 2, kActRelu2 = 3 };
struct ActParams {
  int32_t kind;
  float alpha, beta, limit;  // kActSwigluOai only
};

struct Layout {
  int32_t fmt, E, H, I;
  int32_t Ip;       // FC1 row pairs per expert: I (gated), I / 2 (relu2)
  int32_t G;        // elements per scale byte
  int32_t nC1;      // FC1 chunks per row (H/32)
  int32_t nC2;      // FC2 chunks per row (I/32)
  int32_t nB1;      // FC1 tiles per expert (Ip/32)
  int32_t nB2;      // FC2 tiles per expert (ceil(H/64))
  int32_t nQ1;      // FC1 scale dwords per lane (ceil(H/G/4))
  int32_t nQ2;      // FC2 scale dwords per lane (ceil(I/G/4))
  int32_t csf;      // tiles carry a CSF block (compressed scale format)
  int64_t tile1;    // bytes of one FC1 tile
  int64_t tile2;    // bytes of one FC2 tile
  int64_t w13;      // bytes of an expert's FC1 tiles
  int64_t expert;   // expert stride
  int64_t globals;  // bytes of the globals header
  ActParams act;    // the layer's activation (not part of the byte layout)
};
// The decode kernels take a Layout by value: it stays at 112 bytes (derived
// sizes below are functions, not fields), so their arguments fit the same
// kernel-argument cache lines as before the CSF flag (a larger struct cost
// FC2 0.3 us per launch from a cold cache).
static_assert(sizeof(Layout) == 112, "Layout is passed by value to every kernel");

// Whole prepared buffer.
MOE_HD inline int64_t layout_total(const Layout& L) { return L.globals + L.expert * L.E; }
// Offset of the CSF block in an FC1 / FC2 tile (after the codes and plain scales).
MOE_HD inline int64_t csf_offset1(const Layout& L) { return (int64_t)L.nC1 * 1024 + (int64_t)L.nQ1 * 256; }
MOE_HD inline int64_t csf_offset2(const Layout& L) { return (int64_t)L.nC2 * 1024 + (int64_t)L.nQ2 * 256; }

MOE_HD inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Chunks whose offsets one CSF word holds: 24 (MXFP4), 3 (NVFP4).
MOE_HD inline int32_t csf_chunks_per_word(int32_t fmt) { return fmt == kMXFP4 ? 24 : 3; }

// Bytes of the CSF block of a tile with nC chunks per row: 256 B (64 words)
// per group of chunks.
MOE_HD inline int64_t csf_block_bytes(int32_t fmt, int32_t nC) {
  const int32_t cw = csf_chunks_per_word(fmt);
  return 256 * (int64_t)((nC + cw - 1) / cw);
}

// Returns false when the shape is outside what the layout supports.  W13
// has 2I rows when `gated`, I rows (I a multiple of 64) otherwise; `csf`
// adds the compressed scale blocks.
MOE_HD inline bool make_layout(int32_t fmt, int32_t E, int32_t H, int32_t I, Layout* L, bool gated = true,
                               bool csf = false) {
  if (fmt != kMXFP4 && fmt != kNVFP4) return false;
  if (E <= 0 || H <= 0 || I <= 0 || H % 32 || I % 32) return false;
  if (!gated && I % 64) return false;
  L->Ip = gated ? I : I / 2;
  L->fmt = fmt;
  L->E = E;
  L->H = H;
  L->I = I;
  L->G = fmt == kMXFP4 ? 32 : 16;
  L->nC1 = H / 32;
  L->nC2 = I / 32;
  L->nB1 = L->Ip / 32;
  L->nB2 = (H + 63) / 64;
  L->nQ1 = (H / L->G + 3) / 4;
  L->nQ2 = (I / L->G + 3) / 4;
  L->csf = csf ? 1 : 0;
  L->tile1 = (int64_t)L->nC1 * 1024 + (int64_t)L->nQ1 * 256 + (csf ? csf_block_bytes(fmt, L->nC1) : 0);
  L->tile2 = (int64_t)L->nC2 * 1024 + (int64_t)L->nQ2 * 256 + (csf ? csf_block_bytes(fmt, L->nC2) : 0);
  L->w13 = L->tile1 * L->nB1;
  L->expert = align_up(L->w13 + L->tile2 * L->nB2, 256);
  L->globals = fmt == kNVFP4 ? align_up(8 * (int64_t)E, 256) : 0;
  L->act = ActParams{kActSilu, 0.0f, 0.0f, 0.0f};
  return true;
}

// Logical FC1 row held by lane l of FC1 tile b.
MOE_HD inline int32_t fc1_row(const Layout& L, int32_t b, int32_t l) {
  return l < 32 ? 32 * b + l : L.Ip + 32 * b + (l - 32);
}

MOE_HD inline int64_t fc1_tile_offset(const Layout& L, int32_t e, int32_t b) {
  return L.globals + L.expert * e + L.tile1 * b;
}

MOE_HD inline int64_t fc2_tile_offset(const Layout& L, int32_t e, int32_t hb) {
  return L.globals + L.expert * e + L.w13 + L.tile2 * hb;
}

}  // namespace moe
