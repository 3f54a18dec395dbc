// The element quantizer of the packed format, shared by the codec kernels
// and the fused decode step of the matrix-core attend, so both produce the
// same bytes.  From "KV分组打包：4-bit到底省了多少？" (huhohoo.com/docs/llm/kv-packed-groups),
// section "what a byte holds": per group one float32 scale max|x|/qmax (1 if
// that is 0), codes rint(x/scale) clipped to [-qmax, qmax], stored as code +
// qmax.  Bit-exactness rests on IEEE correctly rounded float32 division
// (-fhip-fp32-correctly-rounded-divide-sqrt), kept denormals and rintf
// rounding half to even, in every translation unit that includes this.
// Internal header.
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {
namespace {

template <int BITS>
struct Codec {
  static constexpr float kQmax = BITS == 4 ? 7.0f : 127.0f;
  static constexpr int kQmaxInt = BITS == 4 ? 7 : 127;
};

// Scale of one group from its largest magnitude.
template <int BITS>
__device__ __forceinline__ float group_scale(float amax) {
  float s = amax / Codec<BITS>::kQmax;
  return s == 0.0f ? 1.0f : s;
}

// Stored (offset) code of one element.
template <int BITS>
__device__ __forceinline__ unsigned stored_code(float x, float s) {
  float c = rintf(x / s);
  c = fminf(fmaxf(c, -Codec<BITS>::kQmax), Codec<BITS>::kQmax);
  return static_cast<unsigned>(static_cast<int>(c) + Codec<BITS>::kQmaxInt);
}

}  // namespace
}  // namespace kvq
