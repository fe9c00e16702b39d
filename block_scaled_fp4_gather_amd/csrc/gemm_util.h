// Device helpers shared by the grouped GEMMs (bf16 and MXFP8 activations):
// direct global -> LDS copies with manual waits, the A ring swizzle, the
// MFMA 32x32 accumulator row map, and the XCD-aware workgroup -> tile map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_char*)p);
}

// Direct global -> LDS copies (global_load_lds_dword[x4]): lane l's bytes at
// `g` land at LDS byte lds + 4 * size_dwords * l.  Written as asm so that the
// compiler does not put a wait for every copy in flight before each LDS read
// (it cannot tell the ring slots apart); the caller waits with vm_wait.  m0,
// which holds the LDS base, is saved and restored.  No memory clobber: a
// copy only writes a ring slot that no LDS access of the current step
// touches, and every read of it comes after vm_wait and a barrier, which the
// compiler keeps in order.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  uint32_t tmp;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(tmp) : "v"(g), "s"(lds));
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  uint32_t tmp;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(tmp) : "v"(g), "s"(lds));
}
// The same for data read once (weights): non-temporal, so that it does not
// displace reused lines in the caches.
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds) {
  uint32_t tmp;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
               : "=&s"(tmp) : "v"(g), "s"(lds));
}
// Wait until at most N vector memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Position of 16-byte chunk c in row r of an A slot.
__device__ __forceinline__ int a_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Row (within the 32x32 block) of accumulator register r of this lane.
__device__ __forceinline__ int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

// Workgroup -> (expert, m-tile, column block) of a grouped GEMM whose experts
// own m-tiles [tile_start[e], tile_start[e + 1]) (tile_expert[t]: the expert
// of m-tile t).  Workgroups are dealt to the 8 XCDs in turn, so consecutive
// ids are remapped to give each XCD a contiguous range of tiles; within it
// the order is expert by expert, column block by column block, with the
// expert's m-tiles innermost: the workgroups that stream the same weight slab
// (same expert and column block) are dispatched together and share it in
// that XCD's L2, and the column blocks of an m-tile share its A rows there.
// Expert e's workgroups are the ids [tile_start[e], tile_start[e + 1]) times
// nblocks, so the expert of id l is tile_expert[l / nblocks]: one load where
// a search over tile_start would take log2(E) dependent ones.  The grid is a
// multiple of 8; ok is false past the last tile.
struct GroupTile {
  int e, gm, nb;
  bool ok;
};
__device__ __forceinline__ GroupTile group_tile(int nblocks, const int* __restrict__ tile_start,
                                                const int* __restrict__ tile_expert, int E) {
  const int per = gridDim.x / 8;
  const int logical = (blockIdx.x % 8) * per + blockIdx.x / 8;
  const int total = tile_start[E];
  if (logical >= total * nblocks) return GroupTile{0, 0, 0, false};
  const int e = tile_expert[logical / nblocks];
  const int t0 = tile_start[e];
  const int nt = tile_start[e + 1] - t0;
  const int local = logical - t0 * nblocks;
  return GroupTile{e, t0 + local % nt, local / nt, true};
}

// Grid of n tiles rounded up to whole XCD rounds (group_tile needs a multiple of 8).
inline unsigned grid8(int64_t n) { return (unsigned)((n + 7) / 8 * 8); }

}  // namespace moe
