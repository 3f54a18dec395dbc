// Pack (quantize + nibble-pack) and dequantize kernels for gfx950.
//
// Format, from "KV分组打包：4-bit到底省了多少？" (huhohoo.com/docs/llm/kv-packed-groups),
// sections "what a byte holds" and "why grouping needs both direction and
// length": per group of `group` elements one float32 scale max|x|/qmax
// (1 if that is 0), codes rint(x/scale) clipped to [-qmax, qmax] and stored
// as code + qmax; 4-bit codes pair up as low | high << 4.  K groups run along
// tokens inside a channel, V groups along features inside a token.  The byte
// order in memory is the block layout of kvq_layout.h.
//
// Packing runs in two passes: one thread per group computes the scale, then
// one thread per stored byte quantizes its one or two elements against the
// scales just written (every byte of the layout is written, padding
// included).
//
// Bit-exactness rests on three properties of this translation unit's build:
// float32 division is IEEE correctly rounded (hipcc's default for HIP,
// requested explicitly with -fhip-fp32-correctly-rounded-divide-sqrt),
// denormals are kept (no flush-to-zero flag), and rintf rounds half to even.
#include "kvq_internal.h"
#include "kvq_layout.h"

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

// K scales: one thread per (head, token group G, channel d), d fastest so
// both the token-row reads and the group-major scale writes coalesce.
template <int BITS>
__global__ __launch_bounds__(256) void pack_k_scales_kernel(const float* __restrict__ x,
                                                            long long BH, Layout L,
                                                            float* __restrict__ scales) {
  const long long tid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tid >= BH * L.kgroups * L.D) return;
  const int d = static_cast<int>(tid % L.D);
  const long long rest = tid / L.D;
  const int g = static_cast<int>(rest % L.kgroups);
  const long long bh = rest / L.kgroups;
  const float* src = x + bh * L.N * static_cast<long long>(L.D) + d;
  const int n1 = min(L.N, (g + 1) * L.group);
  float amax = 0.0f;
  for (int n = g * L.group; n < n1; ++n)
    amax = fmaxf(amax, fabsf(src[static_cast<long long>(n) * L.D]));
  scales[bh * k_scales_per_head(L) + k_scale_index(L, g * L.group, d)] = group_scale<BITS>(amax);
}

// K codes: one thread per stored byte.
template <int BITS>
__global__ __launch_bounds__(256) void pack_k_codes_kernel(const float* __restrict__ x,
                                                           long long BH, Layout L,
                                                           const float* __restrict__ scales,
                                                           uint8_t* __restrict__ codes) {
  const long long per_head = k_code_bytes_per_head(L);
  const long long tid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tid >= BH * per_head) return;
  const long long bh = tid / per_head;
  const long long i = tid % per_head;
  const int blk = static_cast<int>(i / L.kblock_bytes);
  const int r = static_cast<int>(i % L.kblock_bytes);
  const int d = (r / (L.kcols * 8)) * 8 + (r & 7);
  const int j = (r / 8) % L.kcols;
  const float* src = x + bh * L.N * static_cast<long long>(L.D);
  const float* ks = scales + bh * k_scales_per_head(L);
  auto code = [&](int t) -> unsigned {
    if (t >= L.N || d >= L.D) return Codec<BITS>::kQmaxInt;
    return stored_code<BITS>(src[static_cast<long long>(t) * L.D + d], ks[k_scale_index(L, t, d)]);
  };
  const int t0 = blk * kBlockTokens + (BITS == 4 ? 2 * j : j);
  const unsigned byte = BITS == 4 ? (code(t0) | (code(t0 + 1) << 4)) : code(t0);
  codes[tid] = static_cast<uint8_t>(byte);
}

// V scales: one thread per (head, token t < 32 * nblocks, feature group G),
// token fastest so the token-minor scale writes coalesce.
template <int BITS>
__global__ __launch_bounds__(256) void pack_v_scales_kernel(const float* __restrict__ x,
                                                            long long BH, Layout L,
                                                            float* __restrict__ scales) {
  const int tpad = L.nblocks * kBlockTokens;
  const long long tid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tid >= BH * L.vgroups * tpad) return;
  const int tl = static_cast<int>(tid % kBlockTokens);
  long long rest = tid / kBlockTokens;
  const int g = static_cast<int>(rest % L.vgroups);
  rest /= L.vgroups;
  const int blk = static_cast<int>(rest % L.nblocks);
  const long long bh = rest / L.nblocks;
  const int t = blk * kBlockTokens + tl;
  float amax = 0.0f;
  if (t < L.N) {
    const float* src = x + (bh * L.N + t) * static_cast<long long>(L.D);
    const int f1 = min(L.D, (g + 1) * L.group);
    for (int f = g * L.group; f < f1; ++f) amax = fmaxf(amax, fabsf(src[f]));
  }
  scales[bh * v_scales_per_head(L) + v_scale_index(L, t, g * L.group)] = group_scale<BITS>(amax);
}

// V codes: one thread per stored byte.
template <int BITS>
__global__ __launch_bounds__(256) void pack_v_codes_kernel(const float* __restrict__ x,
                                                           long long BH, Layout L,
                                                           const float* __restrict__ scales,
                                                           uint8_t* __restrict__ codes) {
  const long long per_head = v_code_bytes_per_head(L);
  const long long tid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tid >= BH * per_head) return;
  const long long bh = tid / per_head;
  const long long i = tid % per_head;
  const int blk = static_cast<int>(i / L.vblock_bytes);
  const int r = static_cast<int>(i % L.vblock_bytes);
  const int t = blk * kBlockTokens + (r / (L.vcols * 8)) * 8 + (r & 7);
  const int col = (r / 8) % L.vcols;
  unsigned byte;
  if (t >= L.N) {
    byte = BITS == 4 ? Codec<4>::kQmaxInt * 0x11u : Codec<8>::kQmaxInt;
  } else {
    const float* src = x + (bh * L.N + t) * static_cast<long long>(L.D);
    const float* vs = scales + bh * v_scales_per_head(L);
    auto code = [&](int f) -> unsigned {
      const float v = f < L.D ? src[f] : 0.0f;
      return stored_code<BITS>(v, vs[v_scale_index(L, t, f)]);
    };
    byte = BITS == 4 ? (code(2 * col) | (code(2 * col + 1) << 4)) : code(col);
  }
  codes[tid] = static_cast<uint8_t>(byte);
}

// Stored code of element (t, i) given its byte offset within the head.
template <int BITS>
__device__ __forceinline__ int load_code(const uint8_t* head, long long byte, int odd) {
  const unsigned b = head[byte];
  if (BITS == 4) return static_cast<int>(odd ? (b >> 4) : (b & 15u));
  return static_cast<int>(b);
}

// Decode to the original [B][H][N][D] layout, one thread per output element
// (d fastest, so the float32 stores coalesce).  fl32((stored - qmax) * s):
// the integer difference is exact in float32, the multiply rounds once.
template <int BITS, bool K_STYLE>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scales,
                                                      long long BH, Layout L,
                                                      float* __restrict__ out) {
  const long long tid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tid >= BH * L.N * static_cast<long long>(L.D)) return;
  const int d = static_cast<int>(tid % L.D);
  const long long rest = tid / L.D;
  const int n = static_cast<int>(rest % L.N);
  const long long bh = rest / L.N;
  int c;
  float s;
  if (K_STYLE) {
    c = load_code<BITS>(codes + bh * k_code_bytes_per_head(L), k_code_byte(L, n, d), n & 1);
    s = scales[bh * k_scales_per_head(L) + k_scale_index(L, n, d)];
  } else {
    c = load_code<BITS>(codes + bh * v_code_bytes_per_head(L), v_code_byte(L, n, d), d & 1);
    s = scales[bh * v_scales_per_head(L) + v_scale_index(L, n, d)];
  }
  out[tid] = static_cast<float>(c - Codec<BITS>::kQmaxInt) * s;
}

inline unsigned grid_for(long long threads) {
  return static_cast<unsigned>((threads + 255) / 256);
}

template <int BITS>
hipError_t pack_bits(const float* x, long long BH, const Layout& L, bool k_style, uint8_t* codes,
                     float* scales, hipStream_t stream) {
  if (k_style) {
    hipLaunchKernelGGL(pack_k_scales_kernel<BITS>, dim3(grid_for(BH * L.kgroups * L.D)),
                       dim3(256), 0, stream, x, BH, L, scales);
    hipLaunchKernelGGL(pack_k_codes_kernel<BITS>, dim3(grid_for(BH * k_code_bytes_per_head(L))),
                       dim3(256), 0, stream, x, BH, L, scales, codes);
  } else {
    hipLaunchKernelGGL(pack_v_scales_kernel<BITS>,
                       dim3(grid_for(BH * L.vgroups * L.nblocks * kBlockTokens)), dim3(256), 0,
                       stream, x, BH, L, scales);
    hipLaunchKernelGGL(pack_v_codes_kernel<BITS>, dim3(grid_for(BH * v_code_bytes_per_head(L))),
                       dim3(256), 0, stream, x, BH, L, scales, codes);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const float* x, int B, int H, int N, int D, int bits, int group,
                       bool k_style, uint8_t* codes, float* scales, hipStream_t stream) {
  const long long BH = static_cast<long long>(B) * H;
  const Layout L = make_layout(N, D, bits, group);
  return bits == 4 ? pack_bits<4>(x, BH, L, k_style, codes, scales, stream)
                   : pack_bits<8>(x, BH, L, k_style, codes, scales, stream);
}

hipError_t launch_dequant(const uint8_t* codes, const float* scales, int B, int H, int N, int D,
                          int bits, int group, bool k_style, float* out, hipStream_t stream) {
  const long long BH = static_cast<long long>(B) * H;
  const Layout L = make_layout(N, D, bits, group);
  const unsigned grid = grid_for(BH * N * static_cast<long long>(D));
  if (k_style) {
    if (bits == 4)
      hipLaunchKernelGGL((dequant_kernel<4, true>), dim3(grid), dim3(256), 0, stream, codes,
                         scales, BH, L, out);
    else
      hipLaunchKernelGGL((dequant_kernel<8, true>), dim3(grid), dim3(256), 0, stream, codes,
                         scales, BH, L, out);
  } else {
    if (bits == 4)
      hipLaunchKernelGGL((dequant_kernel<4, false>), dim3(grid), dim3(256), 0, stream, codes,
                         scales, BH, L, out);
    else
      hipLaunchKernelGGL((dequant_kernel<8, false>), dim3(grid), dim3(256), 0, stream, codes,
                         scales, BH, L, out);
  }
  return hipGetLastError();
}

}  // namespace kvq
