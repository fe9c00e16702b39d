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
// The W4A8-MX variant (b12x PR #22, Measured table and the sentence on the
// dynamic path: MXFP4 weights with activations quantised to MXFP8, cos
// 0.9990 against an fp32 reference; flashinfer #4285 review of the direct
// micro kernel: one E8M0 scale per 32 K values of the activation):
//  * MXFP8 follows the OCP MX definition: per 32 consecutive values, shared
//    exponent floor(log2(max |v|)) - 8 (8 = exponent of E4M3's largest
//    power of two), clamped to [-127, 127]; every value divided by 2^shared
//    and rounded to nearest-even E4M3, magnitudes above 448 set to 448.
//    A block of zeros (max 0) gets scale byte 0; a block holding a NaN or an
//    infinity gets scale byte 255 (NaN) and every element code 0x7F.
//  * x is quantised per token along H; SiLU(gate) * up per route along I,
//    after FC1's outputs and the product are rounded to fp32 (the fp32
//    intermediate of the pages), so the codes are decided from fp32 values.
//  * Only MXFP4 weights (the scaled products take E8M0 scales).
//
// Other gated activations (flashinfer #4285, reviews of moe_activation.py
// and of the direct micro kernel's activation coverage name gelu_tanh and
// swigluoai_uninterleave with alpha, beta and limit, without formulas):
//  * gelu_tanh(gate) * up with the tanh form of GELU,
//    0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)));
//  * swigluoai: g = min(gate, limit), u = clamp(up, -limit, limit),
//    g * sigmoid(alpha g) * (u + beta), the clamps written as comparisons so
//    that a NaN passes through; gate and up are the separate halves of W13.
//  * relu2 is not gated (b12x #311, commit message on the FP4 quantiser, which
//    keeps relu2 on its exact path because it is not a gated activation; the
//    survey's reading): W13 then has I rows, h_n = x . W13[n], and
//    a_n = max(h_n, 0)^2, a NaN passing through.
//
// Compressed scales (b12x PR #459, "Reduce NVFP4-CSF scale reconstruction
// overhead", commit messages: one-bit MXFP4 and four-bit NVFP4 offsets from a
// row base byte; the scale reconstruction does an exception lookup).  The
// pages give no more than that sentence; the reading here, lossless:
//  * A weight row's scale bytes s[0..n) (one per block along K) are stored
//    as a base byte b and one offset per block, s[j] = b + o[j] as an
//    integer on the byte (UE8M0 exponents for MXFP4, E4M3 codes for NVFP4),
//    with o[j] in [0, 1] (MXFP4, one bit) or [0, 15] (NVFP4, four bits).
//  * b is the smallest byte of the row.  A row whose bytes span more than
//    the offsets reach, or whose smallest byte is 255, is an exception: its
//    base byte is 255 and its offsets 0, and the reader takes its bytes
//    from the uncompressed scales instead.
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

// E4M3 code nearest to v (ties to even code), magnitude capped at 448,
// NaN -> 0x7F.  Works on the value, not its bits: finds the binade, rounds
// the scaled significand, then re-encodes.
uint8_t e4m3_encode(double v) {
  if (std::isnan(v)) return 0x7F;
  const uint8_t sign = std::signbit(v) ? 0x80 : 0x00;
  double a = std::fabs(v);
  if (a > 448.0) a = 448.0;
  int e = 0;
  double m = 0.0;  // significand times 8, an integer after rounding
  if (a >= std::ldexp(1.0, -6)) {
    std::frexp(a, &e);  // a = f * 2^e, f in [0.5, 1)
    e -= 1;             // floor(log2(a))
    m = std::nearbyint(std::ldexp(a, 3 - e));  // in [8, 16]
    if (m == 16.0) {
      m = 8.0;
      e += 1;
    }
    if (e > 8 || (e == 8 && m > 14.0)) {  // above 448 after rounding
      e = 8;
      m = 14.0;
    }
    return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)(m - 8.0));
  }
  m = std::nearbyint(std::ldexp(a, 9));  // subnormal steps of 2^-9, 0..8
  if (m == 8.0) return (uint8_t)(sign | 0x08);  // rounds up to the smallest normal
  return (uint8_t)(sign | (uint8_t)m);
}

// One MXFP8 block of 32 values: codes[32] and the scale byte.
uint8_t mxfp8_block(const float* v, uint8_t* codes) {
  double amax = 0.0;
  bool special = false;
  for (int i = 0; i < 32; ++i) {
    if (!std::isfinite(v[i])) special = true;
    else if (std::fabs((double)v[i]) > amax) amax = std::fabs((double)v[i]);
  }
  if (special) {
    for (int i = 0; i < 32; ++i) codes[i] = 0x7F;
    return 255;
  }
  int shared = -127;
  if (amax > 0.0) {
    int e = 0;
    std::frexp(amax, &e);  // floor(log2(amax)) = e - 1
    shared = e - 1 - 8;
  }
  if (shared < -127) shared = -127;
  if (shared > 127) shared = 127;
  for (int i = 0; i < 32; ++i) codes[i] = e4m3_encode(std::ldexp((double)v[i], -shared));
  return (uint8_t)(shared + 127);
}

double mxfp8_value(uint8_t code, uint8_t scale) {
  return (double)e4m3fn(code) * (double)ue8m0(scale);
}

const int ACT_SILU = 0;
const int ACT_GELU_TANH = 1;
const int ACT_SWIGLUOAI = 2;
const int ACT_RELU2 = 3;  // not gated: one projection of I rows

struct Act {
  int kind;
  double alpha, beta, limit;
};

// The gated activation in the precision T (float for the fp32 oracle,
// double for the others), each operation rounded in T.
template <typename T>
T gated(const Act& a, T g, T u) {
  if (a.kind == ACT_GELU_TANH) {
    const T c = (T)0.7978845608028654;  // sqrt(2 / pi)
    return (T)0.5 * g * ((T)1 + std::tanh(c * (g + (T)0.044715 * g * g * g))) * u;
  }
  if (a.kind == ACT_SWIGLUOAI) {
    const T lim = (T)a.limit;
    const T gc = g > lim ? lim : g;
    const T uc = u > lim ? lim : (u < -lim ? -lim : u);
    return gc / ((T)1 + std::exp(-(T)a.alpha * gc)) * (uc + (T)a.beta);
  }
  return g / ((T)1 + std::exp(-g)) * u;
}

// relu(h)^2; NaN stays NaN.
template <typename T>
T relu2(T h) {
  if (h != h) return h;
  return h > (T)0 ? h * h : (T)0;
}

bool valid_act(int kind) {
  return kind == ACT_SILU || kind == ACT_GELU_TANH || kind == ACT_SWIGLUOAI || kind == ACT_RELU2;
}

// Rows of W13: 2I for the gated activations, I for relu2.
int w13_rows(int act, int I) { return act == ACT_RELU2 ? I : 2 * I; }

// Offset reach of a compressed scale row: 1 (one bit, MXFP4) or 15 (four
// bits, NVFP4).
uint32_t csf_reach(int fmt) { return fmt == FMT_MXFP4 ? 1u : 15u; }

}  // namespace

extern "C" {

// Compressed-scale encoding of one row of n scale bytes: writes the base byte
// and n offsets (one per block, unpacked) and returns 1, or marks the row an
// exception (base 255, offsets 0) and returns 0.  Returns -1 on bad
// arguments.
int oracle_csf_encode(int fmt, const uint8_t* scales, int n, uint8_t* base, uint8_t* offsets) {
  if ((fmt != FMT_MXFP4 && fmt != FMT_NVFP4) || n <= 0 || !scales || !base || !offsets) return -1;
  uint32_t lo = 255u, hi = 0u;
  for (int j = 0; j < n; ++j) {
    if (scales[j] < lo) lo = scales[j];
    if (scales[j] > hi) hi = scales[j];
  }
  if (lo == 255u || hi - lo > csf_reach(fmt)) {
    *base = 255u;
    for (int j = 0; j < n; ++j) offsets[j] = 0u;
    return 0;
  }
  *base = (uint8_t)lo;
  for (int j = 0; j < n; ++j) offsets[j] = (uint8_t)(scales[j] - lo);
  return 1;
}

// The row's scale bytes back from its base and offsets; an exception row
// (base 255) takes them from `plain` (its uncompressed bytes).
int oracle_csf_decode(int fmt, uint8_t base, const uint8_t* offsets, const uint8_t* plain, int n,
                      uint8_t* scales) {
  if ((fmt != FMT_MXFP4 && fmt != FMT_NVFP4) || n <= 0 || !offsets || !plain || !scales) return -1;
  for (int j = 0; j < n; ++j) {
    if (base == 255u) {
      scales[j] = plain[j];
    } else {
      if (offsets[j] > csf_reach(fmt)) return -1;
      scales[j] = (uint8_t)(base + offsets[j]);
    }
  }
  return 0;
}


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
                       float* acc_out, uint16_t* out_bf16, int act, float alpha, float beta,
                       float limit) {
  if (!valid_args(fmt, E, H, I, M, k) || !valid_act(act)) return 1;
  const Act A{act, alpha, beta, limit};
  const int G = block_size(fmt);
  const size_t w13_cb = (size_t)w13_rows(act, I) * (H / 2), w13_sb = (size_t)w13_rows(act, I) * (H / G);
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
      // FC1 and activation: a[n] = f(gate_n, up_n), or relu2(h_n) (not gated).
      for (int n = 0; n < I && act == ACT_RELU2; ++n) {
        float h1 = 0.0f;
        for (int h = 0; h < H; ++h) grow[h] = weight(fmt, c13, s13, gl13, H, n, h);
        for (int h = 0; h < H; ++h) h1 += xf[h] * grow[h];
        a[n] = relu2<float>(h1);
      }
      for (int n = 0; n < I && act != ACT_RELU2; ++n) {
        float gate = 0.0f, up = 0.0f;
        for (int h = 0; h < H; ++h) grow[h] = weight(fmt, c13, s13, gl13, H, n, h);
        for (int h = 0; h < H; ++h) gate += xf[h] * grow[h];
        for (int h = 0; h < H; ++h) grow[h] = weight(fmt, c13, s13, gl13, H, I + n, h);
        for (int h = 0; h < H; ++h) up += xf[h] * grow[h];
        a[n] = gated<float>(A, gate, up);
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
                       double* acc_out, int act, float alpha, float beta, float limit) {
  if (!valid_args(fmt, E, H, I, M, k) || !valid_act(act)) return 1;
  const Act A{act, alpha, beta, limit};
  const int G = block_size(fmt);
  const size_t w13_cb = (size_t)w13_rows(act, I) * (H / 2), w13_sb = (size_t)w13_rows(act, I) * (H / G);
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
          if (act != ACT_RELU2)
            up += xv * weight(fmt, w13_codes + e * w13_cb, w13_scales + e * w13_sb, gl13, H, I + n, h);
        }
        a[n] = act == ACT_RELU2 ? relu2<double>(gate) : gated<double>(A, gate, up);
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

// The activation in fp64 (act: 0 SiLU, 1 gelu_tanh, 2 swigluoai, 3 relu2,
// which takes `gate` as its one input and ignores `up`).
double oracle_activation(int act, double alpha, double beta, double limit, double gate, double up) {
  if (act == ACT_RELU2) return relu2<double>(gate);
  return gated<double>(Act{act, alpha, beta, limit}, gate, up);
}

// MXFP8 quantisation of a [rows][cols] fp32 matrix (cols a multiple of 32):
// codes [rows][cols], scales [rows][cols / 32].
int oracle_mxfp8_quantize(const float* v, int rows, int cols, uint8_t* codes, uint8_t* scales) {
  if (rows < 0 || cols <= 0 || cols % 32) return 1;
  for (int r = 0; r < rows; ++r)
    for (int b = 0; b < cols / 32; ++b)
      scales[(size_t)r * (cols / 32) + b] =
          mxfp8_block(v + (size_t)r * cols + 32 * b, codes + (size_t)r * cols + 32 * b);
  return 0;
}

// Value of an MXFP8 element (E4M3 code times its UE8M0 scale), in fp64.
double oracle_mxfp8_value(uint32_t code, uint32_t scale) {
  return mxfp8_value((uint8_t)code, (uint8_t)scale);
}

// The W4A8-MX layer (MXFP4 weights only): x quantised to MXFP8 per token,
// FC1 dot products in fp64 then rounded to fp32, a = SiLU(gate) * up rounded
// to fp32, then (quant_act != 0) quantised to MXFP8 per route in blocks of 32
// along I, FC2 and the router-weighted sum in fp64.  quant_act = 0 feeds the
// fp32 a to FC2 unquantised (used to check the rest of the chain).  `act`
// and its parameters choose the gated activation, as in the other forms.
int oracle_forward_w4a8(int fmt, int E, int H, int I, int M, int k, const uint8_t* w13_codes,
                        const uint8_t* w13_scales, const uint8_t* w2_codes,
                        const uint8_t* w2_scales, const float* g13, const float* g2,
                        const uint16_t* x, const int64_t* ids, const float* topk_w,
                        int quant_act, double* acc_out, int act, float alpha, float beta,
                        float limit) {
  (void)g13;
  (void)g2;
  if (fmt != FMT_MXFP4 || !valid_args(fmt, E, H, I, M, k) || !valid_act(act)) return 1;
  const Act A{act, alpha, beta, limit};
  const size_t w13_cb = (size_t)w13_rows(act, I) * (H / 2), w13_sb = (size_t)w13_rows(act, I) * (H / 32);
  const size_t w2_cb = (size_t)H * (I / 2), w2_sb = (size_t)H * (I / 32);
  std::vector<float> xf(H), af(I);
  std::vector<uint8_t> xc(H), ac(I), xs(H / 32), as(I / 32);
  std::vector<double> xq(H), aq(I);
  for (int t = 0; t < M; ++t) {
    for (int h = 0; h < H; ++h) xf[h] = bf16_to_f32(x[(size_t)t * H + h]);
    oracle_mxfp8_quantize(xf.data(), 1, H, xc.data(), xs.data());
    for (int h = 0; h < H; ++h) xq[h] = mxfp8_value(xc[h], xs[h / 32]);
    for (int h = 0; h < H; ++h) acc_out[(size_t)t * H + h] = 0.0;
    for (int j = 0; j < k; ++j) {
      const int64_t id = ids[(size_t)t * k + j];
      if (id < 0 || id >= E) continue;
      const int e = (int)id;
      const uint8_t* c13 = w13_codes + (size_t)e * w13_cb;
      const uint8_t* s13 = w13_scales + (size_t)e * w13_sb;
      for (int n = 0; n < I; ++n) {
        double gate = 0.0, up = 0.0;
        for (int h = 0; h < H; ++h) {
          gate += xq[h] * weight(fmt, c13, s13, 1.0f, H, n, h);
          if (act != ACT_RELU2) up += xq[h] * weight(fmt, c13, s13, 1.0f, H, I + n, h);
        }
        const double g = (float)gate, u = (float)up;
        af[n] = (float)(act == ACT_RELU2 ? relu2<double>(g) : gated<double>(A, g, u));
      }
      if (quant_act) {
        oracle_mxfp8_quantize(af.data(), 1, I, ac.data(), as.data());
        for (int n = 0; n < I; ++n) aq[n] = mxfp8_value(ac[n], as[n / 32]);
      } else {
        for (int n = 0; n < I; ++n) aq[n] = af[n];
      }
      const uint8_t* c2 = w2_codes + (size_t)e * w2_cb;
      const uint8_t* s2 = w2_scales + (size_t)e * w2_sb;
      for (int h = 0; h < H; ++h) {
        double y = 0.0;
        for (int n = 0; n < I; ++n) y += aq[n] * weight(fmt, c2, s2, 1.0f, I, h, n);
        acc_out[(size_t)t * H + h] += (double)topk_w[(size_t)t * k + j] * y;
      }
    }
  }
  return 0;
}

}  // extern "C"
