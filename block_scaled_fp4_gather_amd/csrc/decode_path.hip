// Decode-band forward (few tokens): two launches, FC1 then FC2.
//
// Prior art is the two-launch tiny-decode kernel of b12x PR #22 ("rp-native
// tiny-decode kernel for w4a8_mx (M=1)", What section): gate+up dot products
// into an fp32 intermediate, then FC2 with inline SiLU and a router-weighted
// epilogue into the bf16 output, and no grid barrier (its Notes section records
// the grid-barrier variant deadlocking).
//
// On gfx950 a wave's 64 lanes are split as lane = (g, p) = (lane / KL,
// lane % KL): lane p of a group owns 32-element K chunk p of the wave's KL
// chunks, for the rows g + RG*j (RG = 64 / KL row groups, j < T rows per
// lane).  One load instruction then covers KL chunks x 8 consecutive rows of
// the resident layout, whole 128-byte lines, and a lane's activation chunk
// (32 bf16, from LDS where it is staged, else from global memory) is read
// once and reused for its T rows.  The KL partial sums of a row are reduced
// across lanes by a transposing DPP fold inside 16-lane rows (fold_rows),
// which leaves one row sum per lane.  All cross-wave sums stay inside a
// workgroup, in LDS and in a fixed order: no workgroup ever waits for or
// signals another one, and results are bit-reproducible.
//   FC1: one workgroup per (route slot, 64-row tile, block of R rows); its
//        waves split K into slabs; the slab sums meet in LDS, then
//        SiLU(gate)*up is written to the workspace activation.
//   FC2: one workgroup per (block of rows of H, group of whole tokens with
//        at most one route slot per wave); its waves split the group's route
//        slots (experts); the weighted expert sums meet in LDS and are
//        written to the output as bf16, overwriting it.
// FC1 streams each routed expert once per token chunk (at most min(16,
// 64/k) tokens, the chunks on the grid's second dimension) however many of
// the chunk's tokens route to it, FC2 once per token group (one group unless
// a wave would loop over 3 or more route slots; an expert shared by two
// groups is read by both): a
// slot works only if its id is valid and no earlier slot holds the same id
// (b12x PR #22, Notes: re-reading weights per routed row is what limited the
// prior kernel to M=1).  Invalid ids read nothing and add nothing (b12x PR
// #311: commit message on invalid routes and the tiny_decode.py review).
#include <hip/hip_runtime.h>

#include "act.h"
#include "decode.h"
#include "decode_path.h"
#include "layout.h"

namespace moe {

// The route table as one wave sees it: lane l holds slot l (token l / k,
// route l % k).  rid is the expert id, or -1 for an invalid id or a lane past
// the last slot.
struct Routes {
  int rid;
  float w;
};

template <typename IdT>
__device__ __forceinline__ Routes load_routes(const IdT* __restrict__ ids,
                                              const float* __restrict__ tw, int slots, int E) {
  const int l = threadIdx.x & 63;
  Routes r{-1, 0.0f};
  if (l < slots) {
    const int64_t v = (int64_t)ids[l];
    r.rid = (v >= 0 && v < E) ? (int)v : -1;
    if (tw) r.w = tw[l];
  }
  return r;
}

// The same table read in two steps: issue_route_ids loads every lane's id (a
// lane past the last slot reads the last one, 1 <= slots <= 64) and
// finish_route_ids decodes it, so that loads issued in between are in flight
// together with the table's.
template <typename IdT>
__device__ __forceinline__ IdT issue_route_ids(const IdT* __restrict__ ids, int slots) {
  return ids[min((int)(threadIdx.x & 63), slots - 1)];
}

template <typename IdT>
__device__ __forceinline__ Routes finish_route_ids(IdT id, int slots, int E) {
  Routes r{-1, 0.0f};
  if ((int)(threadIdx.x & 63) < slots) {
    const int64_t v = (int64_t)id;
    r.rid = (v >= 0 && v < E) ? (int)v : -1;
  }
  return r;
}

// Expert of slot s when s is the first slot that holds it (else -1), and the
// mask of all slots that hold it.
__device__ __forceinline__ int slot_expert(const Routes& R, int s, uint64_t* mask) {
  const int e = __builtin_amdgcn_readlane(R.rid, s);
  if (e < 0) return -1;
  const uint64_t m = __ballot(R.rid == e);
  if (m & ((1ull << s) - 1ull)) return -1;
  *mask = m;
  return e;
}

__device__ __forceinline__ uint64_t token_routes(uint64_t mask, int t, int k) {
  const uint64_t kmask = k >= 64 ? ~0ull : ((1ull << k) - 1ull);
  return (mask >> (t * k)) & kmask;
}

// DPP lane exchange inside a 16-lane row: partner = lane ^ X for X in
// {1, 3, 7, 15} (quad_perm [1,0,3,2], quad_perm [3,2,1,0], row_half_mirror,
// row_mirror).
template <int X>
__device__ __forceinline__ float dpp_xor(float v) {
  constexpr int ctrl = X == 1 ? 0xB1 : X == 3 ? 0x1B : X == 7 ? 0x141 : 0x140;
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}

template <int M>
__device__ __forceinline__ void fold_stage(float* v, bool upper) {
  // v[0, 2M) -> v[0, M): keep the half selected by this lane's bit, add the
  // partner's copy of the same half (the partner selected the other one).
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const float keep = upper ? v[i + M] : v[i];
    const float send = upper ? v[i] : v[i + M];
    v[i] = keep + dpp_xor<2 * M - 1>(send);
  }
}

template <int X, int T>
__device__ __forceinline__ void fold_plain(float* v) {
#pragma unroll
  for (int j = 0; j < T; ++j) v[j] += dpp_xor<X>(v[j]);
}

// Reduction over the KL lanes of a group (KL in {4, 8, 16}, the group
// aligned inside a 16-lane row) of T partial sums per lane (T a power of two,
// T <= KL): on entry lane p holds v[j] for rows j = 0..T-1; on exit lane p
// returns the full sum of row p % T.  Lane bits at or above log2(T) are
// folded plainly (every value adds lane p ^ (2^(b+1) - 1), which differs from
// p in bit b); the lower bits are folded by transposition: stage m pairs lane
// p with lane p ^ (2m - 1), and each lane keeps the half of its rows whose
// bit m matches its own.
template <int KL, int T>
__device__ __forceinline__ float fold_rows(float* v, int p) {
  if (KL >= 16 && T <= 8) fold_plain<15, T>(v);
  if (KL >= 8 && T <= 4) fold_plain<7, T>(v);
  if (KL >= 4 && T <= 2) fold_plain<3, T>(v);
  if (T <= 1) fold_plain<1, T>(v);
  if (T >= 8) fold_stage<4>(v, (p & 4) != 0);
  if (T >= 4) fold_stage<2>(v, (p & 2) != 0);
  if (T >= 2) fold_stage<1>(v, (p & 1) != 0);
  return v[0];
}

// Block scale(s) of chunk c from the lane's scale dword of that row.
template <int FMT>
__device__ __forceinline__ f32x2_t chunk_scale(uint32_t dword, int c) {
  if (FMT == kMXFP4) {
    const float s = mx_scale(dword, c);
    return f32x2_t{s, s};
  }
  return e4m3x2_to_f32(dword, (c & 1) != 0);
}

// Dot product of one 32-element unit with 32 bf16 activations (16 dwords),
// with the block scale(s) applied to the partial sums.
template <int FMT>
__device__ __forceinline__ float unit_dot(const u32x4 q, const uint32_t* a, f32x2_t sc) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float pa = 0.0f, pb = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    bf16x2_t wv[4];
    fp4x8_to_bf16(w[d], wv);  // elements 8d .. 8d+7
    float acc = d < 2 ? pa : pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(wv[i], as_bf16x2(a[4 * d + i]), acc, false);
    if (d < 2)
      pa = acc;
    else
      pb = acc;
  }
  if (FMT == kMXFP4) return (pa + pb) * sc.x;
  return fmaf(pa, sc.x, pb * sc.y);
}

// Same against an activation held as two bf16 planes (a = hi + lo); the
// unit is decoded once for both.
template <int FMT>
__device__ __forceinline__ float unit_dot2(const u32x4 q, const uint32_t* hi, const uint32_t* lo,
                                           f32x2_t sc) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float pa = 0.0f, pb = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    bf16x2_t wv[4];
    fp4x8_to_bf16(w[d], wv);
    float acc = d < 2 ? pa : pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_amdgcn_fdot2_f32_bf16(wv[i], as_bf16x2(hi[4 * d + i]), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(wv[i], as_bf16x2(lo[4 * d + i]), acc, false);
    }
    if (d < 2)
      pa = acc;
    else
      pb = acc;
  }
  if (FMT == kMXFP4) return (pa + pb) * sc.x;
  return fmaf(pa, sc.x, pb * sc.y);
}

__device__ __forceinline__ void load_chunk16(const uint16_t* p, uint32_t* d) {
  const u32x4* q = (const u32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = q[i];
    d[4 * i] = v.x;
    d[4 * i + 1] = v.y;
    d[4 * i + 2] = v.z;
    d[4 * i + 3] = v.w;
  }
}

// Copies n16 16-byte words from global to LDS with all threads of the
// workgroup (no barrier; the caller synchronises before reading).
__device__ __forceinline__ void stage_lds(const void* src, void* dst, int n16) {
  const u32x4* s = (const u32x4*)src;
  u32x4* d = (u32x4*)dst;
  for (int i = threadIdx.x; i < n16; i += blockDim.x) d[i] = s[i];
}

__device__ __forceinline__ void lds_chunk16(const uint16_t* p, uint32_t* d) {
  const u32x4* q = (const u32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = q[i];
    d[4 * i] = v.x;
    d[4 * i + 1] = v.y;
    d[4 * i + 2] = v.z;
    d[4 * i + 3] = v.w;
  }
}

// FC1: one workgroup per (route slot, 64-row tile, block of R rows): R/2 gate
// rows and their R/2 up rows.  Wave w covers chunks [w*KL, w*KL + KL) (and
// further groups of W*KL chunks if K is longer); lane (g, p) = (lane / KL,
// lane % KL) owns chunk w*KL + p of the block rows q = g + RG*j, j < T, so
// its activation chunk is read once and reused for T rows.  The activations
// of the slot's own token are staged in LDS while the route lookup is in
// flight.  With EARLY the route ids and the activations are loaded together
// and the first chunk group's weights are issued ahead of the barrier that
// publishes the staged activations.  Measured on MI355X against staging
// first and the barrier first: FC1 3-6% faster on E512/H2560/I320 (4 chunk
// lanes, 80 chunks of K) and E288/H4096/I512 (4 lanes, 128 chunks), 3-4%
// slower on E256/H7168/I256 (224 chunks) with 4 lanes and with 8, so the
// launch takes it for 4 chunk lanes over at most 128 chunks.
template <int FMT, int KL, int R, bool CSF, bool EARLY, typename IdT>
__global__ void __launch_bounds__(1024)
    fc1_kernel(const uint8_t* __restrict__ prep, const Layout L, const uint16_t* __restrict__ x,
               const IdT* __restrict__ ids, const int M_all, const int k, const int mc,
               uint16_t* __restrict__ act_hi, uint16_t* __restrict__ act_lo) {
  constexpr int SPD = FMT == kMXFP4 ? 4 : 2;  // chunks per scale dword
  constexpr int RG = 64 / KL;                 // row groups of a wave
  constexpr int T = R / RG;                   // rows per lane
  constexpr int NB = 64 / R;                  // blocks per tile
  extern __shared__ u32x4 lds_raw[];
  // Token chunk blockIdx.y: tokens c0 .. c0 + M - 1 (mc per chunk, at most 64
  // route slots, one per lane of the route table), whose activations, route
  // slots and activation rows are contiguous; experts are deduplicated
  // within the chunk.
  const int c0 = blockIdx.y * mc;
  const int M = min(mc, M_all - c0);
  x += (int64_t)c0 * L.H;
  ids += (int64_t)c0 * k;
  act_hi += (int64_t)c0 * k * L.I;
  act_lo += (int64_t)c0 * k * L.I;
  uint16_t* xs = (uint16_t*)lds_raw;                // [H] activations of token t0
  float* part = (float*)(xs + align_up(L.H, 64));  // [token index][16 waves][R rows]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int p = lane % KL, g = lane / KL;
  // Workgroup id = ((tl / 8) NB + blk) 8 + tl % 8 for tile tl = s nB1 + b: the
  // NB blocks of a tile, which share its scale blocks, have ids 8 apart, so
  // round-robin dispatch over the 8 XCDs puts them on one XCD's L2.  The
  // grid covers the tiles rounded up to a multiple of 8.
  const int blk = (int)(blockIdx.x >> 3) % NB;
  const int tl = (int)(blockIdx.x >> 3) / NB * 8 + (int)(blockIdx.x & 7);
  const int b = tl % L.nB1;
  const int s = tl / L.nB1;
  if (s >= M * k) return;  // a slot past the last chunk's tokens, or a padding tile
  const int t0 = s / k;  // the slot's own token routes to the slot's expert
  const int ngroups = (L.nC1 + W * KL - 1) / (W * KL);

  Routes R_;
  if constexpr (EARLY) {
    const IdT id = issue_route_ids(ids, M * k);
    stage_lds(x + (int64_t)t0 * L.H, xs, L.H / 8);
    R_ = finish_route_ids(id, M * k, L.E);
  } else {
    stage_lds(x + (int64_t)t0 * L.H, xs, L.H / 8);
    R_ = load_routes(ids, (const float*)nullptr, M * k, L.E);
  }
  uint64_t mask = 0;
  const int e = slot_expert(R_, s, &mask);
  if (e < 0) return;  // same decision in every wave of the workgroup
  const uint8_t* tile = prep + fc1_tile_offset(L, e, b);
  const uint8_t* sbase = tile + (int64_t)L.nC1 * 1024;
  const uint8_t* csf = tile + csf_offset1(L);  // compressed scales (CSF block)

  int m = 0;
  for (int t = 0; t < M; ++t) m += token_routes(mask, t, k) != 0;
  for (int i = threadIdx.x; i < m * 16 * R; i += blockDim.x) part[i] = 0.0f;
  if constexpr (!EARLY) __syncthreads();

  for (int grp = 0; grp < ngroups; ++grp) {
    const int c = (grp * W + wave) * KL + p;
    const bool cv = c < L.nC1;
    const int cc = min(c, L.nC1 - 1);
    u32x4 q[T];
    uint32_t sd[T];
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const int qr = g + RG * j;  // block row: R/2 gate rows, then R/2 up rows
      const int row = (qr < R / 2 ? 0 : 32 - R / 2) + blk * (R / 2) + qr;
      q[j] = __builtin_nontemporal_load((const u32x4*)(tile + (int64_t)cc * 1024 + row * 16));
      if (CSF)
        sd[j] = csf_load<FMT>(csf, row, cc);
      else
        sd[j] = __builtin_nontemporal_load((const uint32_t*)(sbase + (cc / SPD) * 256 + row * 4));
    }
    if (EARLY && grp == 0) __syncthreads();  // staged activations and zeroed sums from here on
    // The chunk scale word of row j: the plain word, or rebuilt from the CSF
    // word where it is used (an exception row, base 255, reads its plain word).
    auto sword = [&](int j) -> uint32_t {
      if (!CSF) return sd[j];
      if (!csf_exception(sd[j])) return csf_word<FMT>(sd[j], cc);
      const int qr = g + RG * j;
      const int row = (qr < R / 2 ? 0 : 32 - R / 2) + blk * (R / 2) + qr;
      return *(const uint32_t*)(sbase + (cc / SPD) * 256 + row * 4);
    };
    int ti = 0;
    for (int t = 0; t < M; ++t) {
      if (!token_routes(mask, t, k)) continue;
      uint32_t xc[16];
      if (t == t0)
        lds_chunk16(xs + 32 * cc, xc);
      else
        load_chunk16(x + (int64_t)t * L.H + 32 * cc, xc);
      float v[T];
#pragma unroll
      for (int j = 0; j < T; ++j) v[j] = cv ? unit_dot<FMT>(q[j], xc, chunk_scale<FMT>(sword(j), cc)) : 0.0f;
      const float r = fold_rows<KL, T>(v, p);
      if (p < T) part[(ti * 16 + wave) * R + g + RG * p] += r;
      ++ti;
    }
  }
  __syncthreads();
  const float g13 = FMT == kNVFP4 ? ((const float*)prep)[e] : 1.0f;
  int ti = 0;
  for (int t = 0; t < M; ++t) {
    const uint64_t tm = token_routes(mask, t, k);
    if (!tm) continue;
    if (ti % W == wave && lane < R / 2) {
      float gate = 0.0f, up = 0.0f;
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        gate += part[(ti * 16 + w) * R + lane];
        up += part[(ti * 16 + w) * R + R / 2 + lane];
      }
      gate *= g13;
      up *= g13;
      // a = hi + lo in two bf16 planes: 16 significant bits for FC2's bf16
      // dot products.
      const int64_t at = (int64_t)(t * k + __builtin_ctzll(tm)) * L.I + 32 * b + blk * (R / 2) + lane;
      auto put = [&](int64_t o, float a) {
        const uint16_t hi = f32_to_bf16_rne(a);
        act_hi[o] = hi;
        act_lo[o] = f32_to_bf16_rne(a - __uint_as_float((uint32_t)hi << 16));
      };
      if (L.act.kind == kActRelu2) {  // not gated: both halves are outputs
        put(at, relu2(gate));
        put(at + L.Ip, relu2(up));
      } else {
        put(at, gated_act(L.act, gate, up));
      }
    }
    ++ti;
  }
}

// FC2: one workgroup per (block of R rows of H, token group); its waves
// split the group's route slots.  Lane (g, p) owns chunk c0 + p of the
// expert's block rows q = g + RG*j, j < T.  With STAGE, the activations of
// every route slot of the group are staged in LDS while the route lookup is
// in flight.
template <int FMT, int KL, int R, int CI, bool STAGE, bool CSF, typename IdT>
__global__ void __launch_bounds__(64 * fc2_max_waves(KL))
    fc2_kernel(const uint8_t* __restrict__ prep, const Layout L, const IdT* __restrict__ ids,
               const float* __restrict__ tw, const int M_all, const int k, const int tg,
               const uint16_t* __restrict__ act_hi, const uint16_t* __restrict__ act_lo,
               uint16_t* __restrict__ out) {
  constexpr int SPD = FMT == kMXFP4 ? 4 : 2;
  constexpr int RG = 64 / KL;
  constexpr int T = R / RG;
  extern __shared__ u32x4 lds_raw[];
  // Token group blockIdx.y: tokens g0 .. g0 + M - 1 (tg per group), whose
  // route slots, activation rows and output rows are contiguous; the group
  // is a call of its own over those tokens.
  const int g0 = blockIdx.y * tg;
  const int M = min(tg, M_all - g0);
  ids += (int64_t)g0 * k;
  tw += (int64_t)g0 * k;
  act_hi += (int64_t)g0 * k * L.I;
  act_lo += (int64_t)g0 * k * L.I;
  out += (int64_t)g0 * L.H;
  const int slots = M * k;
  float* part = (float*)lds_raw;                           // [token][16 waves][R rows]
  uint16_t* as = (uint16_t*)(part + M * 16 * R);           // [slot][hi | lo][I]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int p = lane % KL, g = lane / KL;
  const int row0 = blockIdx.x * R;  // first row of H
  const int hb = row0 / 64;
  if (STAGE) {
    // hi and lo planes are separate buffers of slots x I bf16 each
    for (int i = threadIdx.x; i < slots * L.I / 8; i += blockDim.x) {
      const int r = i / (L.I / 8), c = i % (L.I / 8);
      ((u32x4*)(as + (int64_t)r * 2 * L.I))[c] = ((const u32x4*)(act_hi + (int64_t)r * L.I))[c];
      ((u32x4*)(as + (int64_t)r * 2 * L.I + L.I))[c] = ((const u32x4*)(act_lo + (int64_t)r * L.I))[c];
    }
  }
  const Routes R_ = load_routes(ids, tw, slots, L.E);
  for (int i = threadIdx.x; i < M * 16 * R; i += blockDim.x) part[i] = 0.0f;
  __syncthreads();

  for (int s = wave; s < slots; s += W) {
    uint64_t mask = 0;
    const int e = slot_expert(R_, s, &mask);
    if (e < 0) continue;
    const uint8_t* tile = prep + fc2_tile_offset(L, e, hb);
    const uint8_t* sbase = tile + (int64_t)L.nC2 * 1024;
    const uint8_t* csf = tile + csf_offset2(L);  // compressed scales (CSF block)
    const float g2 = FMT == kNVFP4 ? ((const float*)prep)[L.E + e] : 1.0f;
    // CI groups of KL chunks per pass, all their loads issued together
    for (int c0 = 0; c0 < L.nC2; c0 += CI * KL) {
      u32x4 q[CI][T];
      uint32_t sd[CI][T];
#pragma unroll
      for (int ci = 0; ci < CI; ++ci) {
        const int cc = min(c0 + ci * KL + p, L.nC2 - 1);
#pragma unroll
        for (int j = 0; j < T; ++j) {
          const int row = row0 % 64 + g + RG * j;  // tile rows past H are zero padding
          q[ci][j] = __builtin_nontemporal_load((const u32x4*)(tile + (int64_t)cc * 1024 + row * 16));
          if (CSF)
            sd[ci][j] = csf_load<FMT>(csf, row, cc);
          else
            sd[ci][j] = __builtin_nontemporal_load((const uint32_t*)(sbase + (cc / SPD) * 256 + row * 4));
        }
      }
      for (int t = 0; t < M; ++t) {
        uint64_t tm = token_routes(mask, t, k);
        if (!tm) continue;
        const int r = t * k + __builtin_ctzll(tm);
        float wsum = 0.0f;  // duplicate routes of a token share one FC2 result
        while (tm) {
          const int j = __builtin_ctzll(tm);
          tm &= tm - 1;
          wsum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(R_.w), t * k + j));
        }
        float v[T];
#pragma unroll
        for (int ci = 0; ci < CI; ++ci) {
          const int c = c0 + ci * KL + p;
          const bool cv = c < L.nC2;
          const int cc = min(c, L.nC2 - 1);
          uint32_t ah[16], al[16];
          if (STAGE) {
            lds_chunk16(as + (int64_t)r * 2 * L.I + 32 * cc, ah);
            lds_chunk16(as + (int64_t)r * 2 * L.I + L.I + 32 * cc, al);
          } else {
            load_chunk16(act_hi + (int64_t)r * L.I + 32 * cc, ah);
            load_chunk16(act_lo + (int64_t)r * L.I + 32 * cc, al);
          }
#pragma unroll
          for (int j = 0; j < T; ++j) {
            // the chunk scale word: plain, or rebuilt from the CSF word (an
            // exception row, base 255, reads its plain word here)
            uint32_t word = sd[ci][j];
            if (CSF)
              word = !csf_exception(word) ? csf_word<FMT>(word, cc)
                                          : *(const uint32_t*)(sbase + (cc / SPD) * 256 + (row0 % 64 + g + RG * j) * 4);
            const f32x2_t sc = chunk_scale<FMT>(word, cc);
            const float d = cv ? unit_dot2<FMT>(q[ci][j], ah, al, sc) : 0.0f;
            v[j] = ci == 0 ? d : v[j] + d;
          }
        }
        const float y = fold_rows<KL, T>(v, p);
        if (p < T) part[(t * 16 + wave) * R + g + RG * p] += (y * g2) * wsum;
      }
    }
  }
  __syncthreads();
  const int h = row0 + lane;
  if (lane >= R || h >= L.H) return;
  for (int t = wave; t < M; t += W) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < 16; ++w) v += part[(t * 16 + w) * R + lane];
    out[(int64_t)t * L.H + h] = f32_to_bf16_rne(v);
  }
}

template <int FMT, int KL, typename IdT>
hipError_t launch_fc1(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                      const IdT* ids, uint16_t* act_hi, uint16_t* act_lo, int R, hipStream_t st) {
  const int mc = M < decode_max_tokens(k) ? M : decode_max_tokens(k);  // tokens per chunk
  const int slots = mc * k;
  const int groups = (L.nC1 + KL - 1) / KL;
  const int waves = groups < kMaxWaves ? groups : kMaxWaves;
  const bool big = R == 32;
  const size_t lds = (size_t)fc1_lds_bytes(L, mc, R);
  const int64_t tiles8 = ((int64_t)slots * L.nB1 + 7) / 8 * 8;  // see fc1_kernel's workgroup ids
  const dim3 grid((unsigned)(tiles8 * (64 / R)), (unsigned)((M + mc - 1) / mc)), block(64 * waves);
  const bool early = KL == 4 && L.nC1 <= 128;
#define MOE_FC1_E(RR, CC, EE)                                                                                   \
  hipLaunchKernelGGL((fc1_kernel<FMT, KL, RR, CC, EE, IdT>), grid, block, lds, st, prep, L, x, ids, M, k, mc, \
                     act_hi, act_lo)
#define MOE_FC1(RR, CC)           \
  do {                            \
    if constexpr (KL == 4) {      \
      if (early)                  \
        MOE_FC1_E(RR, CC, true);  \
      else                        \
        MOE_FC1_E(RR, CC, false); \
    } else {                      \
      MOE_FC1_E(RR, CC, false);   \
    }                             \
  } while (0)
  if (big) {
    if constexpr (KL == 16) {  // 8 rows per lane: no registers left for compressed scales
      if (L.csf) return hipErrorInvalidValue;  // valid_shape rejects this shape first
      MOE_FC1(32, false);
    } else {
      if (L.csf)
        MOE_FC1(32, true);
      else
        MOE_FC1(32, false);
    }
  } else {
    if (L.csf)
      MOE_FC1(16, true);
    else
      MOE_FC1(16, false);
  }
#undef MOE_FC1
#undef MOE_FC1_E
  return hipGetLastError();
}

template <int FMT, int KL, int R, int CI, typename IdT>
hipError_t launch_fc2_ci(const Layout& L, const uint8_t* prep, int M, int k, const IdT* ids,
                         const float* tw, const uint16_t* ah, const uint16_t* al, uint16_t* out,
                         hipStream_t st) {
  // Tokens per workgroup (the groups form the grid's second dimension).
  // When a wave would loop over 3 or more route slots, whole tokens whose
  // slots fit one per wave (at least one token), in larger groups while the
  // grid exceeds 1280 workgroups; else every token in one group.  Measured
  // on MI355X: FC2 16.2 -> 12.6 us on E512 at 40 routes, 19.2 -> 16.2 us on
  // E288 at M = 5; 2 slots per wave stay faster in one group.
  const int maxw = fc2_max_waves(KL);
  const int64_t nhb = (L.H + R - 1) / R;
  const int mc = decode_max_tokens(k);  // a group's route table fits one wave
  int tg = M < mc ? M : mc;
  if ((int64_t)tg * k > 2 * maxw) {
    const int tg0 = k >= maxw ? 1 : maxw / k;
    tg = tg0;
    while (tg < M && tg + tg0 <= mc && nhb * ((M + tg - 1) / tg) > 1280) tg += tg0;
    if (tg > M) tg = M;
  }
  const int slots = tg * k;
  const int waves = slots < maxw ? slots : maxw;
  const size_t act_bytes = (size_t)slots * L.I * 4;
  const size_t part_bytes = (size_t)tg * 16 * R * sizeof(float);
  const bool stage = act_bytes <= kStageActBytes && part_bytes + act_bytes <= kMaxLdsBytes;
  const size_t lds = part_bytes + (stage ? act_bytes : 0);
  const dim3 grid((unsigned)((L.H + R - 1) / R), (unsigned)((M + tg - 1) / tg)), block(64 * waves);
#define MOE_FC2(SS, CC)                                                                                  \
  hipLaunchKernelGGL((fc2_kernel<FMT, KL, R, CI, SS, CC, IdT>), grid, block, lds, st, prep, L, ids, tw, M, k, tg, \
                     ah, al, out)
  constexpr bool csf_ok = csf_shape_ok(KL, R, CI);
  if (L.csf && !csf_ok) return hipErrorInvalidValue;  // valid_shape rejects this shape first
  if (stage) {
    if constexpr (csf_ok) {
      if (L.csf) MOE_FC2(true, true);
    }
    if (!L.csf) MOE_FC2(true, false);
  } else {
    if constexpr (csf_ok) {
      if (L.csf) MOE_FC2(false, true);
    }
    if (!L.csf) MOE_FC2(false, false);
  }
#undef MOE_FC2
  return hipGetLastError();
}

template <int FMT, int KL, int R, typename IdT>
hipError_t launch_fc2_r(const Layout& L, const uint8_t* prep, int M, int k, const IdT* ids,
                        const float* tw, const uint16_t* ah, const uint16_t* al, uint16_t* out,
                        hipStream_t st) {
  if constexpr (KL == 8) {
    if (fc2_chunk_groups(L) == 2) return launch_fc2_ci<FMT, KL, R, 2, IdT>(L, prep, M, k, ids, tw, ah, al, out, st);
  }
  return launch_fc2_ci<FMT, KL, R, 1, IdT>(L, prep, M, k, ids, tw, ah, al, out, st);
}

template <int FMT, int KL, typename IdT>
hipError_t launch_fc2(const Layout& L, const uint8_t* prep, int M, int k, const IdT* ids,
                      const float* tw, const uint16_t* ah, const uint16_t* al, uint16_t* out,
                      int R, hipStream_t st) {
  if (R == 32) return launch_fc2_r<FMT, KL, 32, IdT>(L, prep, M, k, ids, tw, ah, al, out, st);
  if constexpr (KL == 4) {
    return launch_fc2_r<FMT, KL, 16, IdT>(L, prep, M, k, ids, tw, ah, al, out, st);
  } else {
    if (R == 16) return launch_fc2_r<FMT, KL, 16, IdT>(L, prep, M, k, ids, tw, ah, al, out, st);
    return launch_fc2_r<FMT, KL, 8, IdT>(L, prep, M, k, ids, tw, ah, al, out, st);
  }
}

template <int FMT, typename IdT>
hipError_t launch_decode_fmt(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                             const IdT* ids, const float* tw, uint16_t* out, uint8_t* ws,
                             const DecodeWs& W, const DecodeShape& sh, int phases, hipStream_t st) {
  uint16_t* act_hi = (uint16_t*)(ws + W.act_hi);
  uint16_t* act_lo = (uint16_t*)(ws + W.act_lo);
  if (phases & 1) {
    hipError_t err;
    if (sh.kl1 == 4)
      err = launch_fc1<FMT, 4, IdT>(L, prep, x, M, k, ids, act_hi, act_lo, sh.r1, st);
    else if (sh.kl1 == 8)
      err = launch_fc1<FMT, 8, IdT>(L, prep, x, M, k, ids, act_hi, act_lo, sh.r1, st);
    else
      err = launch_fc1<FMT, 16, IdT>(L, prep, x, M, k, ids, act_hi, act_lo, sh.r1, st);
    if (err != hipSuccess) return err;
  }
  if (phases & 2) {
    const int kl2 = fc2_chunk_lanes(L);
    if (kl2 == 4) return launch_fc2<FMT, 4, IdT>(L, prep, M, k, ids, tw, act_hi, act_lo, out, sh.r2, st);
    if (kl2 == 8) return launch_fc2<FMT, 8, IdT>(L, prep, M, k, ids, tw, act_hi, act_lo, out, sh.r2, st);
    return launch_fc2<FMT, 16, IdT>(L, prep, M, k, ids, tw, act_hi, act_lo, out, sh.r2, st);
  }
  return hipSuccess;
}

template <typename IdT>
hipError_t launch_decode(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                         const IdT* ids, const float* tw, uint16_t* out, uint8_t* ws,
                         const DecodeWs& W, const DecodeShape& sh, int phases, hipStream_t st) {
  if (L.fmt == kMXFP4)
    return launch_decode_fmt<kMXFP4, IdT>(L, prep, x, M, k, ids, tw, out, ws, W, sh, phases, st);
  return launch_decode_fmt<kNVFP4, IdT>(L, prep, x, M, k, ids, tw, out, ws, W, sh, phases, st);
}

template hipError_t launch_decode<int32_t>(const Layout&, const uint8_t*, const uint16_t*, int, int,
                                           const int32_t*, const float*, uint16_t*, uint8_t*,
                                           const DecodeWs&, const DecodeShape&, int, hipStream_t);
template hipError_t launch_decode<int64_t>(const Layout&, const uint8_t*, const uint16_t*, int, int,
                                           const int64_t*, const float*, uint16_t*, uint8_t*,
                                           const DecodeWs&, const DecodeShape&, int, hipStream_t);

}  // namespace moe
