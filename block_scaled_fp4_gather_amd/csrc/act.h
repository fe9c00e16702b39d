// The gated activations of the FC1 epilogues, a = f(gate, up) in fp32.
// The pages name SiLU (b12x PR #22, What: FC2 applies SiLU inline),
// gelu_tanh and swigluoai_uninterleave with alpha, beta and limit (flashinfer
// #4285, the review of moe_activation.py and of the direct micro kernel's
// activation coverage) without formulas; these are the standard ones:
//   silu:       gate * sigmoid(gate) * up
//   gelu_tanh:  0.5 * gate * (1 + tanh(sqrt(2/pi) * (gate + 0.044715 gate^3))) * up
//   swigluoai:  g = min(gate, limit), u = clamp(up, -limit, limit),
//               g * sigmoid(alpha * g) * (u + beta)
// (gate and up are separate halves of W13, not interleaved).  The clamps
// are comparisons, so a NaN passes through them.  relu2 is not gated:
// max(h, 0)^2 of each FC1 output on its own (relu2()).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "layout.h"

namespace moe {

// The activation of kind KIND (a compile-time constant, so that an
// epilogue unrolled over many values holds only its own arithmetic);
// kActRelu2 takes g alone.
template <int KIND>
__device__ __forceinline__ float act_of(const ActParams& p, float g, float u) {
  if constexpr (KIND == kActGeluTanh) {
    const float z = 0.7978845608028654f * (g + 0.044715f * g * g * g);
    const float th = 1.0f - 2.0f / (1.0f + __expf(2.0f * z));  // tanh(z), saturating to +-1
    return 0.5f * g * (1.0f + th) * u;
  } else if constexpr (KIND == kActSwigluOai) {
    const float gc = g > p.limit ? p.limit : g;
    const float uc = u > p.limit ? p.limit : (u < -p.limit ? -p.limit : u);
    return gc / (1.0f + __expf(-p.alpha * gc)) * (uc + p.beta);
  } else if constexpr (KIND == kActRelu2) {
    return g != g ? g : (g > 0.0f ? g * g : 0.0f);
  } else {
    return g / (1.0f + __expf(-g)) * u;
  }
}

// Calls f(std::integral_constant<int, kind>) for the runtime kind (one
// branch per epilogue, not per value).
template <typename F>
__device__ __forceinline__ void with_act_kind(int kind, F&& f) {
  switch (kind) {
    case kActGeluTanh: f(std::integral_constant<int, kActGeluTanh>{}); break;
    case kActSwigluOai: f(std::integral_constant<int, kActSwigluOai>{}); break;
    case kActRelu2: f(std::integral_constant<int, kActRelu2>{}); break;
    default: f(std::integral_constant<int, kActSilu>{}); break;
  }
}

// The gated activation of the runtime kind p.kind (a branch per value; for
// epilogues with few values).
__device__ __forceinline__ float gated_act(const ActParams& p, float g, float u) {
  float a = 0.0f;
  with_act_kind(p.kind, [&](auto kind) { a = act_of<decltype(kind)::value>(p, g, u); });
  return a;
}

// relu(h)^2, NaN passing through.
__device__ __forceinline__ float relu2(float h) { return act_of<kActRelu2>(ActParams{}, h, 0.0f); }

}  // namespace moe
