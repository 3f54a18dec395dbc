// Pack (quantize + nibble-pack) and dequantize kernels for gfx950.
//
// Format, from "KV分组打包：4-bit到底省了多少？" (huhohoo.com/docs/llm/kv-packed-groups),
// sections "what a byte holds" and "why grouping needs both direction and
// length": per group of `group` elements one float32 scale max|x|/qmax
// (1 if that is 0), codes rint(x/scale) clipped to [-qmax, qmax] and stored
// as code + qmax; 4-bit codes pair up as low | high << 4.  K groups run along
// tokens inside a channel, V groups along features inside a token.
//
// Bit-exactness rests on three properties of this translation unit's build:
// float32 division is IEEE correctly rounded (hipcc's default for HIP,
// requested explicitly with -fhip-fp32-correctly-rounded-divide-sqrt),
// denormals are kept (no flush-to-zero flag), and rintf rounds half to even.
#include "kvq_internal.h"

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

// K-style: one thread per (b*h, group index G, channel d).  Consecutive
// threads take consecutive channels, so each of the `group` token reads is
// one coalesced row segment.  The thread writes its group's codes
// (group*BITS/8 bytes) into channel d's row and one scale.
template <int BITS>
__global__ __launch_bounds__(256) void pack_k_kernel(const float* __restrict__ x, long long BH,
                                                     int N, int D, int group, int ngroups,
                                                     uint8_t* __restrict__ codes,
                                                     float* __restrict__ scales) {
  const long long tid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tid >= BH * ngroups * D) return;
  const int d = static_cast<int>(tid % D);
  const long long rest = tid / D;
  const int g = static_cast<int>(rest % ngroups);
  const long long bh = rest / ngroups;
  const float* src = x + bh * N * static_cast<long long>(D) + d;
  const int n0 = g * group;
  const int n1 = min(N, n0 + group);

  float amax = 0.0f;
  for (int n = n0; n < n1; ++n) amax = fmaxf(amax, fabsf(src[static_cast<long long>(n) * D]));
  const float s = group_scale<BITS>(amax);

  const long long row = bh * D + d;
  scales[row * ngroups + g] = s;
  const long long row_bytes = static_cast<long long>(ngroups) * group * BITS / 8;
  uint8_t* dst = codes + row * row_bytes + static_cast<long long>(n0) * BITS / 8;
  for (int t = 0; t < group; t += 2) {
    const int n = n0 + t;
    const float x0 = n < N ? src[static_cast<long long>(n) * D] : 0.0f;
    const float x1 = n + 1 < N ? src[static_cast<long long>(n + 1) * D] : 0.0f;
    const unsigned c0 = stored_code<BITS>(x0, s);
    const unsigned c1 = stored_code<BITS>(x1, s);
    if (BITS == 4) {
      dst[t / 2] = static_cast<uint8_t>(c0 | (c1 << 4));
    } else {
      dst[t] = static_cast<uint8_t>(c0);
      dst[t + 1] = static_cast<uint8_t>(c1);
    }
  }
}

// V-style: one thread per (token row, group index G); the group is a
// contiguous run of features.
template <int BITS>
__global__ __launch_bounds__(256) void pack_v_kernel(const float* __restrict__ x, long long rows,
                                                     int D, int group, int ngroups,
                                                     uint8_t* __restrict__ codes,
                                                     float* __restrict__ scales) {
  const long long tid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tid >= rows * ngroups) return;
  const int g = static_cast<int>(tid % ngroups);
  const long long row = tid / ngroups;
  const float* src = x + row * D;
  const int f0 = g * group;
  const int f1 = min(D, f0 + group);

  float amax = 0.0f;
  for (int f = f0; f < f1; ++f) amax = fmaxf(amax, fabsf(src[f]));
  const float s = group_scale<BITS>(amax);

  scales[row * ngroups + g] = s;
  const long long row_bytes = static_cast<long long>(ngroups) * group * BITS / 8;
  uint8_t* dst = codes + row * row_bytes + static_cast<long long>(f0) * BITS / 8;
  for (int t = 0; t < group; t += 2) {
    const int f = f0 + t;
    const float x0 = f < D ? src[f] : 0.0f;
    const float x1 = f + 1 < D ? src[f + 1] : 0.0f;
    const unsigned c0 = stored_code<BITS>(x0, s);
    const unsigned c1 = stored_code<BITS>(x1, s);
    if (BITS == 4) {
      dst[t / 2] = static_cast<uint8_t>(c0 | (c1 << 4));
    } else {
      dst[t] = static_cast<uint8_t>(c0);
      dst[t + 1] = static_cast<uint8_t>(c1);
    }
  }
}

// Stored code of element `i` of a packed row.
template <int BITS>
__device__ __forceinline__ int load_code(const uint8_t* row, long long i) {
  if (BITS == 4) {
    const unsigned b = row[i >> 1];
    return static_cast<int>((i & 1) ? (b >> 4) : (b & 15u));
  }
  return static_cast<int>(row[i]);
}

// Decode to the original [B][H][N][D] layout, one thread per output element
// (d fastest, so the float32 stores coalesce).  fl32((stored - qmax) * s):
// the integer difference is exact in float32, the multiply rounds once.
template <int BITS, bool K_STYLE>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scales,
                                                      long long BH, int N, int D, int group,
                                                      int ngroups, float* __restrict__ out) {
  const long long tid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tid >= BH * N * static_cast<long long>(D)) return;
  const int d = static_cast<int>(tid % D);
  const long long rest = tid / D;
  const int n = static_cast<int>(rest % N);
  const long long bh = rest / N;
  const long long row_bytes = static_cast<long long>(ngroups) * group * BITS / 8;
  long long row;
  int i;
  if (K_STYLE) {
    row = bh * D + d;
    i = n;
  } else {
    row = bh * N + n;
    i = d;
  }
  const int c = load_code<BITS>(codes + row * row_bytes, i);
  const float s = scales[row * ngroups + i / group];
  out[tid] = static_cast<float>(c - Codec<BITS>::kQmaxInt) * s;
}

inline unsigned grid_for(long long threads) {
  return static_cast<unsigned>((threads + 255) / 256);
}

}  // namespace

hipError_t launch_pack(const float* x, int B, int H, int N, int D, int bits, int group,
                       bool k_style, uint8_t* codes, float* scales, hipStream_t stream) {
  const long long BH = static_cast<long long>(B) * H;
  if (k_style) {
    const int ngroups = (N + group - 1) / group;
    const unsigned grid = grid_for(BH * ngroups * D);
    if (bits == 4)
      hipLaunchKernelGGL(pack_k_kernel<4>, dim3(grid), dim3(256), 0, stream, x, BH, N, D, group,
                         ngroups, codes, scales);
    else
      hipLaunchKernelGGL(pack_k_kernel<8>, dim3(grid), dim3(256), 0, stream, x, BH, N, D, group,
                         ngroups, codes, scales);
  } else {
    const int ngroups = (D + group - 1) / group;
    const long long rows = BH * N;
    const unsigned grid = grid_for(rows * ngroups);
    if (bits == 4)
      hipLaunchKernelGGL(pack_v_kernel<4>, dim3(grid), dim3(256), 0, stream, x, rows, D, group,
                         ngroups, codes, scales);
    else
      hipLaunchKernelGGL(pack_v_kernel<8>, dim3(grid), dim3(256), 0, stream, x, rows, D, group,
                         ngroups, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const float* scales, int B, int H, int N, int D,
                          int bits, int group, bool k_style, float* out, hipStream_t stream) {
  const long long BH = static_cast<long long>(B) * H;
  const int ngroups = k_style ? (N + group - 1) / group : (D + group - 1) / group;
  const unsigned grid = grid_for(BH * N * static_cast<long long>(D));
  if (k_style) {
    if (bits == 4)
      hipLaunchKernelGGL((dequant_kernel<4, true>), dim3(grid), dim3(256), 0, stream, codes,
                         scales, BH, N, D, group, ngroups, out);
    else
      hipLaunchKernelGGL((dequant_kernel<8, true>), dim3(grid), dim3(256), 0, stream, codes,
                         scales, BH, N, D, group, ngroups, out);
  } else {
    if (bits == 4)
      hipLaunchKernelGGL((dequant_kernel<4, false>), dim3(grid), dim3(256), 0, stream, codes,
                         scales, BH, N, D, group, ngroups, out);
    else
      hipLaunchKernelGGL((dequant_kernel<8, false>), dim3(grid), dim3(256), 0, stream, codes,
                         scales, BH, N, D, group, ngroups, out);
  }
  return hipGetLastError();
}

}  // namespace kvq
