// CPU oracle for the block-scaled FP4 mixture-of-experts layer.
//
// TEST INFRASTRUCTURE ONLY.  Plain, slow, single-threaded C++ that states what
// the layer computes, element by element, in the order the pages describe it.
// It shares no code, header, table or helper with the HIP library; only the
// test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
//
// What it follows:
//  * The layer: per token, gather the top-k routed experts, FC1 (gate and up
//    dot products of the bf16 activations with the FP4 W13 rows) into fp32,
//    SiLU(gate) * up, FC2 (the down projection), router-weighted sum into a
//    bf16 output.  b12x PR #22, "rp-native tiny-decode kernel for w4a8_mx
//    (M=1)", What section (FC1 and FC2 bullets) and its sequence diagram.
//  * Invalid route ids neither read any expert nor contribute: b12x PR #311,
//    commit message on the FC2-only endpoint (invalid routes carry an
//    exact-zero effective weight), and its review of tiny_decode.py, which
//    asks that invalid routes be kept out of both the loads and the stored
//    sums; flashinfer PR #4285 review of the direct micro kernel's narrow FC2
//    paths: a zero weight does not remove a NaN read from unset storage, so
//    invalid routes are skipped, never multiplied by zero.
//  * Weights are native E2M1 nibbles with block scales, not requantised:
//    b12x PR #459, "Reduce NVFP4-CSF scale reconstruction overhead", commit
//    messages (native E2M1, UE8M0 scales, FP32 calibration).
//  * One final rounding of the fp32 token sum to bf16: b12x PR #311, commit
//    message on the prefill fused-sum epilogue (reduce into an fp32 token
//    accumulator, cast once).
//
// Readings where the pages are silent (each is listed with its reason in the
// design notes):
//  * E2M1 values are the OCP MX table +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}; code 8 is -0.
//  * Element 2b of a row sits in the low nibble of byte b, element 2b+1 in
//    the high nibble.
//  * UE8M0 byte b is 2^(b-127); b = 255 is NaN.
//  * E4M3 is the "fn" variant: no infinities, S.1111.111 is NaN, max 448,
//    subnormals (m/8) * 2^-6.
//  * NVFP4 dequant is (code * block scale) * global, each product rounded to
//    fp32; the global is a multiplier, one per expert per matrix.
//  * W13 rows [0, I) are gate, [I, 2I) are up.
//  * Router weights are applied after FC2 and are used as given.
//  * Duplicate ids within a token are separate routes.
//  * A token with no valid route gives +0.
//
// Build: g++ -O2 -ffp-contract=off -shared -fPIC (no fast-math, no FMA
// contraction, so every product and sum is one IEEE fp32 rounding in the
// order written).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

const int FMT_MXFP4 = 1;
const int FMT_NVFP4 = 2;

int block_size(int fmt) { return fmt == FMT_MXFP4 ? 32 : 16; }

float e2m1(uint32_t nibble) {
  // Magnitudes of the eight non-negative codes, in code order.
  static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  float v = mag[nibble & 7u];
  return (nibble & 8u) ? -v : v;
}

float ue8m0(uint32_t b) {
  b &= 0xFFu;
  if (b == 255u) return std::nanf("");
  return std::ldexp(1.0f, (int)b - 127);
}

float e4m3fn(uint32_t b) {
  b &= 0xFFu;
  uint32_t s = b >> 7, e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 15u && m == 7u) return std::nanf("");
  if (e == 0u)
    v = std::ldexp((float)m, -9);           // (m/8) * 2^-6
  else
    v = std::ldexp((float)(8u + m), (int)e - 10);  // (1 + m/8) * 2^(e-7)
  return s ? -v : v;
}

float block_scale(int fmt, uint32_t b) { return fmt == FMT_MXFP4 ? ue8m0(b) : e4m3fn(b); }

float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

uint16_t f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

// Dequantised element (row, col) of one expert matrix with `cols` columns.
float weight(int fmt, const uint8_t* codes, const uint8_t* scales, float global, int cols,
             int row, int col) {
  const uint8_t byte = codes[(size_t)row * (cols / 2) + col / 2];
  const uint32_t nib = (col & 1) ? (byte >> 4) : (byte & 15u);
  const int G = block_size(fmt);
  const float s = block_scale(fmt, scales[(size_t)row * (cols / G) + col / G]);
  float d = e2m1(nib) * s;
  if (fmt == FMT_NVFP4) d = d * global;
  return d;
}

bool valid_args(int fmt, int E, int H, int I, int M, int k) {
  if (fmt != FMT_MXFP4 && fmt != FMT_NVFP4) return false;
  const int G = block_size(fmt);
  return E > 0 && H > 0 && I > 0 && M >= 0 && k > 0 && H % G == 0 && I % G == 0;
}

}  // namespace

extern "C" {

float oracle_e2m1(uint32_t nibble) { return e2m1(nibble); }
float oracle_ue8m0(uint32_t b) { return ue8m0(b); }
float oracle_e4m3(uint32_t b) { return e4m3fn(b); }
float oracle_bf16_to_f32(uint16_t h) { return bf16_to_f32(h); }
uint16_t oracle_f32_to_bf16(float f) { return f32_to_bf16(f); }

// Dequantise one [rows][cols] matrix (one expert's W13 or W2) into fp32.
int oracle_dequant(int fmt, const uint8_t* codes, const uint8_t* scales, float global, int rows,
                   int cols, float* out) {
  if (fmt != FMT_MXFP4 && fmt != FMT_NVFP4) return 1;
  if (cols % block_size(fmt) != 0) return 1;
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c)
      out[(size_t)r * cols + c] = weight(fmt, codes, scales, global, cols, r, c);
  return 0;
}

// The layer in fp32.  ids are int64 so both id widths of the library fit.
// acc_out [M][H] receives the fp32 token sums, out_bf16 [M][H] their bf16.
int oracle_forward_f32(int fmt, int E, int H, int I, int M, int k, const uint8_t* w13_codes,
                       const uint8_t* w13_scales, const uint8_t* w2_codes,
                       const uint8_t* w2_scales, const float* g13, const float* g2,
                       const uint16_t* x, const int64_t* ids, const float* topk_w,
                       float* acc_out, uint16_t* out_bf16) {
  if (!valid_args(fmt, E, H, I, M, k)) return 1;
  const int G = block_size(fmt);
  const size_t w13_cb = (size_t)2 * I * (H / 2), w13_sb = (size_t)2 * I * (H / G);
  const size_t w2_cb = (size_t)H * (I / 2), w2_sb = (size_t)H * (I / G);
  std::vector<float> xf(H), grow(H), a(I), acc(H), w2row(I);
  for (int t = 0; t < M; ++t) {
    for (int h = 0; h < H; ++h) xf[h] = bf16_to_f32(x[(size_t)t * H + h]);
    for (int h = 0; h < H; ++h) acc[h] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int64_t id = ids[(size_t)t * k + j];
      if (id < 0 || id >= E) continue;  // invalid route: no read, no contribution
      const int e = (int)id;
      const uint8_t* c13 = w13_codes + (size_t)e * w13_cb;
      const uint8_t* s13 = w13_scales + (size_t)e * w13_sb;
      const uint8_t* c2 = w2_codes + (size_t)e * w2_cb;
      const uint8_t* s2 = w2_scales + (size_t)e * w2_sb;
      const float gl13 = fmt == FMT_NVFP4 ? g13[e] : 1.0f;
      const float gl2 = fmt == FMT_NVFP4 ? g2[e] : 1.0f;
      // FC1 and activation: a[n] = silu(gate_n) * up_n.
      for (int n = 0; n < I; ++n) {
        float gate = 0.0f, up = 0.0f;
        for (int h = 0; h < H; ++h) grow[h] = weight(fmt, c13, s13, gl13, H, n, h);
        for (int h = 0; h < H; ++h) gate += xf[h] * grow[h];
        for (int h = 0; h < H; ++h) grow[h] = weight(fmt, c13, s13, gl13, H, I + n, h);
        for (int h = 0; h < H; ++h) up += xf[h] * grow[h];
        a[n] = gate / (1.0f + std::exp(-gate)) * up;
      }
      // FC2 and router-weighted combine.
      const float wt = topk_w[(size_t)t * k + j];
      for (int h = 0; h < H; ++h) {
        float y = 0.0f;
        for (int n = 0; n < I; ++n) w2row[n] = weight(fmt, c2, s2, gl2, I, h, n);
        for (int n = 0; n < I; ++n) y += a[n] * w2row[n];
        acc[h] += wt * y;
      }
    }
    for (int h = 0; h < H; ++h) {
      if (acc_out) acc_out[(size_t)t * H + h] = acc[h];
      if (out_bf16) out_bf16[(size_t)t * H + h] = f32_to_bf16(acc[h]);
    }
  }
  return 0;
}

// The same layer in fp64 (dequantised values are exact in fp32, so only the
// dot products, the SiLU and the sums differ).  For tiny shapes.
int oracle_forward_f64(int fmt, int E, int H, int I, int M, int k, const uint8_t* w13_codes,
                       const uint8_t* w13_scales, const uint8_t* w2_codes,
                       const uint8_t* w2_scales, const float* g13, const float* g2,
                       const uint16_t* x, const int64_t* ids, const float* topk_w,
                       double* acc_out) {
  if (!valid_args(fmt, E, H, I, M, k)) return 1;
  const int G = block_size(fmt);
  const size_t w13_cb = (size_t)2 * I * (H / 2), w13_sb = (size_t)2 * I * (H / G);
  const size_t w2_cb = (size_t)H * (I / 2), w2_sb = (size_t)H * (I / G);
  std::vector<double> a(I);
  for (int t = 0; t < M; ++t) {
    for (int h = 0; h < H; ++h) acc_out[(size_t)t * H + h] = 0.0;
    for (int j = 0; j < k; ++j) {
      const int64_t id = ids[(size_t)t * k + j];
      if (id < 0 || id >= E) continue;
      const int e = (int)id;
      const float gl13 = fmt == FMT_NVFP4 ? g13[e] : 1.0f;
      const float gl2 = fmt == FMT_NVFP4 ? g2[e] : 1.0f;
      for (int n = 0; n < I; ++n) {
        double gate = 0.0, up = 0.0;
        for (int h = 0; h < H; ++h) {
          const double xv = bf16_to_f32(x[(size_t)t * H + h]);
          gate += xv * weight(fmt, w13_codes + e * w13_cb, w13_scales + e * w13_sb, gl13, H, n, h);
          up += xv * weight(fmt, w13_codes + e * w13_cb, w13_scales + e * w13_sb, gl13, H, I + n, h);
        }
        a[n] = gate / (1.0 + std::exp(-gate)) * up;
      }
      for (int h = 0; h < H; ++h) {
        double y = 0.0;
        for (int n = 0; n < I; ++n)
          y += a[n] * weight(fmt, w2_codes + e * w2_cb, w2_scales + e * w2_sb, gl2, I, h, n);
        acc_out[(size_t)t * H + h] += (double)topk_w[(size_t)t * k + j] * y;
      }
    }
  }
  return 0;
}

}  // extern "C"
