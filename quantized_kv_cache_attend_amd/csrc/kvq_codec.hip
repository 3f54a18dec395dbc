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
// Packing works per (head, 32-token block) when D <= kStageMaxD: a workgroup
// stages the block's 32 x D inputs in LDS with coalesced loads, computes the
// block's scales (V always; K when the group divides 32, so its groups lie in
// the block) and then writes every stored byte of the block (padding
// included) from LDS.  Otherwise, and for K scales of longer groups, two
// plain passes run: one thread per group computes the scale, then one thread
// per stored byte quantizes its one or two elements against the scales just
// written.
//
// Bit-exactness rests on three properties of this translation unit's build:
// float32 division is IEEE correctly rounded (hipcc's default for HIP,
// requested explicitly with -fhip-fp32-correctly-rounded-divide-sqrt),
// denormals are kept (no flush-to-zero flag), and rintf rounds half to even.
#include "kvq_internal.h"
#include "kvq_layout.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

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

// ---- block-staged packing --------------------------------------------------
// Largest head dim staged through LDS: 32 x (D + 1) floats plus the block's
// scales stay under 64 KB.
constexpr int kStageMaxD = 256;

// Stage tokens t0 .. t0 + nt - 1 (all D values, one contiguous run of
// memory) into tile[tl * (D + 1) + f]; the pad word keeps column reads of
// 32 rows on distinct banks.
__device__ __forceinline__ void stage_block(const float* __restrict__ src, int nt, int D,
                                            float* tile) {
  const int n = nt * D;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int tl = i / D;
    tile[tl * (D + 1) + (i - tl * D)] = src[i];
  }
}

// V: scales and codes of one (head, block).  LDS: tile, then the block's
// scales [group][32 tokens].
template <int BITS>
__global__ __launch_bounds__(256) void pack_v_block_kernel(const float* __restrict__ x,
                                                           Layout L, float* __restrict__ scales,
                                                           uint8_t* __restrict__ codes) {
  extern __shared__ float lds[];
  const long long bh = blockIdx.x / L.nblocks;
  const int blk = static_cast<int>(blockIdx.x % L.nblocks);
  const int t0 = blk * kBlockTokens;
  const int nt = min(kBlockTokens, L.N - t0);
  const int stride = L.D + 1;
  float* tile = lds;
  float* sc = lds + kBlockTokens * stride;
  stage_block(x + (bh * L.N + t0) * static_cast<long long>(L.D), nt, L.D, tile);
  __syncthreads();
  // One thread per (group G, token tl), token fastest: the token-minor scale
  // writes coalesce.  Tokens >= N get scale 1, the scale of an all-zero group.
  float* hs = scales + bh * v_scales_per_head(L) + static_cast<long long>(blk) * L.vgroups * kBlockTokens;
  for (int i = threadIdx.x; i < L.vgroups * kBlockTokens; i += blockDim.x) {
    const int G = i / kBlockTokens, tl = i % kBlockTokens;
    float amax = 0.0f;
    if (tl < nt) {
      const int f1 = min(L.D, (G + 1) * L.group);
      for (int f = G * L.group; f < f1; ++f) amax = fmaxf(amax, fabsf(tile[tl * stride + f]));
    }
    const float sv = group_scale<BITS>(amax);
    sc[i] = sv;
    hs[i] = sv;
  }
  __syncthreads();
  uint8_t* dst = codes + bh * v_code_bytes_per_head(L) + blk * L.vblock_bytes;
  for (int r = threadIdx.x; r < L.vblock_bytes; r += blockDim.x) {
    const int tl = (r / (L.vcols * 8)) * 8 + (r & 7);
    const int col = (r / 8) % L.vcols;
    unsigned byte;
    if (tl >= nt) {
      byte = BITS == 4 ? Codec<4>::kQmaxInt * 0x11u : Codec<8>::kQmaxInt;
    } else {
      auto code = [&](int f) -> unsigned {
        const float v = f < L.D ? tile[tl * stride + f] : 0.0f;
        return stored_code<BITS>(v, sc[(f / L.group) * kBlockTokens + tl]);
      };
      byte = BITS == 4 ? (code(2 * col) | (code(2 * col + 1) << 4)) : code(col);
    }
    dst[r] = static_cast<uint8_t>(byte);
  }
}

// K: codes of one (head, block); with kLocalScales (group divides 32) also
// the block's scales, else they come from pack_k_scales_kernel.  LDS: tile,
// then the block's scales [group in block][D].
template <int BITS, bool kLocalScales>
__global__ __launch_bounds__(256) void pack_k_block_kernel(const float* __restrict__ x,
                                                           Layout L, float* __restrict__ scales,
                                                           uint8_t* __restrict__ codes) {
  extern __shared__ float lds[];
  const long long bh = blockIdx.x / L.nblocks;
  const int blk = static_cast<int>(blockIdx.x % L.nblocks);
  const int t0 = blk * kBlockTokens;
  const int nt = min(kBlockTokens, L.N - t0);
  const int stride = L.D + 1;
  float* tile = lds;
  float* sk = lds + kBlockTokens * stride;
  float* hs = scales + bh * k_scales_per_head(L);
  stage_block(x + (bh * L.N + t0) * static_cast<long long>(L.D), nt, L.D, tile);
  __syncthreads();
  if (kLocalScales) {
    // One thread per (group gi of the block, channel d), channel fastest.
    // Only groups holding a token < N have a scale row.
    const int groups = kBlockTokens / L.group;
    for (int i = threadIdx.x; i < groups * L.D; i += blockDim.x) {
      const int gi = i / L.D, d = i - gi * L.D;
      const int tl0 = gi * L.group;
      if (tl0 >= nt) continue;
      const int tl1 = min(nt, tl0 + L.group);
      float amax = 0.0f;
      for (int tl = tl0; tl < tl1; ++tl) amax = fmaxf(amax, fabsf(tile[tl * stride + d]));
      const float s = group_scale<BITS>(amax);
      sk[i] = s;
      hs[k_scale_index(L, t0 + tl0, d)] = s;
    }
    __syncthreads();
  }
  uint8_t* dst = codes + bh * k_code_bytes_per_head(L) + blk * L.kblock_bytes;
  for (int r = threadIdx.x; r < L.kblock_bytes; r += blockDim.x) {
    const int d = (r / (L.kcols * 8)) * 8 + (r & 7);
    const int j = (r / 8) % L.kcols;
    auto code = [&](int tl) -> unsigned {
      if (tl >= nt || d >= L.D) return Codec<BITS>::kQmaxInt;
      const float s = kLocalScales ? sk[(tl / L.group) * L.D + d]
                                   : hs[k_scale_index(L, t0 + tl, d)];
      return stored_code<BITS>(tile[tl * stride + d], s);
    };
    const int tl = BITS == 4 ? 2 * j : j;
    const unsigned byte = BITS == 4 ? (code(tl) | (code(tl + 1) << 4)) : code(tl);
    dst[r] = static_cast<uint8_t>(byte);
  }
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
// Grid: x over the N * D elements of one head (32-bit index arithmetic),
// y * z over the heads.
template <int BITS, bool K_STYLE>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scales,
                                                      long long BH, Layout L,
                                                      float* __restrict__ out) {
  const unsigned e = blockIdx.x * 256u + threadIdx.x;
  const long long bh = static_cast<long long>(blockIdx.z) * gridDim.y + blockIdx.y;
  if (bh >= BH || e >= static_cast<unsigned>(L.N) * static_cast<unsigned>(L.D)) return;
  const int n = static_cast<int>(e / static_cast<unsigned>(L.D));
  const int d = static_cast<int>(e - static_cast<unsigned>(n) * static_cast<unsigned>(L.D));
  const long long tid = bh * L.N * static_cast<long long>(L.D) + e;
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

// The same decode, four consecutive features of one token per thread (D a
// multiple of 4; code, scale and output arrays 4-, 16- and 16-byte
// aligned): one 16-byte store, K's four code bytes in one 4-byte load and
// its four scales in one 16-byte load.
template <int BITS, bool K_STYLE>
__global__ __launch_bounds__(256) void dequant4_kernel(const uint8_t* __restrict__ codes,
                                                       const float* __restrict__ scales,
                                                       long long BH, Layout L,
                                                       float* __restrict__ out) {
  const unsigned e = blockIdx.x * 256u + threadIdx.x;  // quad index inside the head
  const long long bh = static_cast<long long>(blockIdx.z) * gridDim.y + blockIdx.y;
  const unsigned quads = static_cast<unsigned>(L.D) / 4;
  if (bh >= BH || e >= static_cast<unsigned>(L.N) * quads) return;
  const int n = static_cast<int>(e / quads);
  const int d = static_cast<int>(e - static_cast<unsigned>(n) * quads) * 4;
  constexpr int kQ = Codec<BITS>::kQmaxInt;
  int c[4];
  float s[4];
  if (K_STYLE) {
    // channels d .. d+3 sit in one 4-byte half of an 8-byte run
    const unsigned w = *reinterpret_cast<const unsigned*>(
        codes + bh * k_code_bytes_per_head(L) + k_code_byte(L, n, d));
    const int sh = BITS == 4 ? 4 * (n & 1) : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c[i] = static_cast<int>((w >> (8 * i + sh)) & (BITS == 4 ? 15u : 255u));
    const float4 sc = *reinterpret_cast<const float4*>(
        scales + bh * k_scales_per_head(L) + k_scale_index(L, n, d));
    s[0] = sc.x;
    s[1] = sc.y;
    s[2] = sc.z;
    s[3] = sc.w;
  } else {
    const uint8_t* head = codes + bh * v_code_bytes_per_head(L);
    const float* vs = scales + bh * v_scales_per_head(L);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = load_code<BITS>(head, v_code_byte(L, n, d + i), (d + i) & 1);
      s[i] = vs[v_scale_index(L, n, d + i)];
    }
  }
  float4 o;
  o.x = static_cast<float>(c[0] - kQ) * s[0];
  o.y = static_cast<float>(c[1] - kQ) * s[1];
  o.z = static_cast<float>(c[2] - kQ) * s[2];
  o.w = static_cast<float>(c[3] - kQ) * s[3];
  *reinterpret_cast<float4*>(out + (bh * L.N + n) * static_cast<long long>(L.D) + d) = o;
}

inline unsigned grid_for(long long threads) {
  return static_cast<unsigned>((threads + 255) / 256);
}

// ---- growing cache --------------------------------------------------------
// A decode step reads the cached K/V and appends the new position
// ("给长前缀列一张有单位的资源账本", "prefill and decode").  Here the cache
// after n tokens holds exactly the packed form of those n tokens
// zero-padded to the layout's capacity, i.e. what the pack kernels give for
// that input: an empty cache is all zero codes with scale 1 (the all-zero
// group of the format), V groups lie inside one token so a new token's V is
// packed on its own, and a K group spans `group` tokens of one channel, so
// the open group (the one holding token n - 1 when the group is not full)
// is requantized from float32 on every append, with the K values of its
// earlier tokens taken from the tail the appends keep.

// Empty state: every stored code the zero code, every scale 1.
__global__ __launch_bounds__(256) void cache_clear_kernel(uint8_t* __restrict__ kc, long long nkc,
                                                          float* __restrict__ ks, long long nks,
                                                          uint8_t* __restrict__ vc, long long nvc,
                                                          float* __restrict__ vs, long long nvs,
                                                          uint8_t zero_code) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  const long long first = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (long long i = first; i < nkc; i += stride) kc[i] = zero_code;
  for (long long i = first; i < nvc; i += stride) vc[i] = zero_code;
  for (long long i = first; i < nks; i += stride) ks[i] = 1.0f;
  for (long long i = first; i < nvs; i += stride) vs[i] = 1.0f;
}

// Append tokens [N, N + T) of every head.  Threads [0, BH*ng*D): one K
// group of one channel each (head, touched group gi < ng, channel d; d
// fastest), ng = the number of token groups the new tokens touch; the rest:
// one V group (head, new token, feature group) each.  Only the first
// touched group reads the tail (its tokens below N).  The tokens of the new
// open group are written to the tail by the thread of the last group when
// no other thread of its channel reads the tail in the same launch (it is
// the first group itself, or the first group starts at N); otherwise
// append_tail_kernel writes them after this kernel.  Groups of up to
// kRegGroup elements are loaded into registers in one go (independent
// loads, one memory round trip); longer groups are walked element by
// element.
constexpr int kRegGroup = 32;

template <int BITS>
__global__ __launch_bounds__(256) void append_kernel(const float* __restrict__ k_new,
                                                     const float* __restrict__ v_new,
                                                     long long BH, Layout L, int N, int T,
                                                     int ng, bool tail_here,
                                                     uint8_t* __restrict__ k_codes,
                                                     float* __restrict__ k_scales,
                                                     uint8_t* __restrict__ v_codes,
                                                     float* __restrict__ v_scales,
                                                     float* __restrict__ k_tail) {
  const long long tid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const long long nk = BH * ng * L.D;
  const int n1 = N + T;
  const int g = L.group;
  constexpr int kStep = BITS == 4 ? 2 : 1;  // tokens (K) or features (V) per byte
  constexpr unsigned kZero = Codec<BITS>::kQmaxInt;
  if (tid < nk) {
    const long long D = L.D;
    const int d = static_cast<int>(tid % D);
    const long long rest = tid / D;
    const int gi = static_cast<int>(rest % ng);
    const long long bh = rest / ng;
    const int g0 = (N / g + gi) * g;             // first token of this group
    const float* src = k_new + bh * T * D + d;
    float* tail = k_tail + bh * g * D + d;
    const int cnt = min(g0 + g, n1) - g0;        // tokens of the group that hold values
    const int ncode = min(g0 + g, L.nblocks * kBlockTokens) - g0;  // ... that have codes
    const bool write_tail = tail_here && n1 % g != 0 && gi == ng - 1;
    const int t_tail = max(N, g0);               // first token of the new tail (if written)
    float* scale = k_scales + bh * k_scales_per_head(L) + k_scale_index(L, g0, d);
    uint8_t* codes = k_codes + bh * k_code_bytes_per_head(L);
    // K of token g0 + i (its tail slot is i, g0 being a multiple of g).
    auto value = [&](int i) -> float {
      const int t = g0 + i;
      return t < N ? tail[i * D] : src[(t - N) * D];
    };
    if (g <= kRegGroup) {
      float x[kRegGroup];
#pragma unroll
      for (int i = 0; i < kRegGroup; ++i) x[i] = i < cnt ? value(i) : 0.0f;
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < kRegGroup; ++i) amax = fmaxf(amax, fabsf(x[i]));
      const float s = group_scale<BITS>(amax);
      *scale = s;
#pragma unroll
      for (int i = 0; i < kRegGroup; i += kStep) {
        if (i < ncode) {
          unsigned byte = i < cnt ? stored_code<BITS>(x[i], s) : kZero;
          if (BITS == 4) byte |= (i + 1 < cnt ? stored_code<BITS>(x[i + 1], s) : kZero) << 4;
          codes[k_code_byte(L, g0 + i, d)] = static_cast<uint8_t>(byte);
        }
      }
      if (write_tail) {
#pragma unroll
        for (int i = 0; i < kRegGroup; ++i)
          if (i < cnt && g0 + i >= t_tail) tail[i * D] = x[i];
      }
      return;
    }
    float amax = 0.0f;
    for (int i = 0; i < cnt; ++i) amax = fmaxf(amax, fabsf(value(i)));
    const float s = group_scale<BITS>(amax);
    *scale = s;
    auto code = [&](int i) -> unsigned { return i < cnt ? stored_code<BITS>(value(i), s) : kZero; };
    for (int i = 0; i < ncode; i += kStep) {
      const unsigned byte = BITS == 4 ? (code(i) | (code(i + 1) << 4)) : code(i);
      codes[k_code_byte(L, g0 + i, d)] = static_cast<uint8_t>(byte);
    }
    if (write_tail)
      for (int t = t_tail; t < n1; ++t) tail[(t - g0) * D] = src[(t - N) * D];
    return;
  }
  const long long i = tid - nk;
  if (i >= BH * T * L.vgroups) return;
  const int G = static_cast<int>(i % L.vgroups);
  const long long rest = i / L.vgroups;
  const int j = static_cast<int>(rest % T);
  const long long bh = rest / T;
  const int t = N + j;
  const float* src = v_new + (bh * T + j) * static_cast<long long>(L.D);
  const int f0 = G * g;
  const int cnt = min(L.D, f0 + g) - f0;  // features of the group inside D
  v_scales += bh * v_scales_per_head(L) + v_scale_index(L, t, f0);
  uint8_t* codes = v_codes + bh * v_code_bytes_per_head(L);
  if (g <= kRegGroup) {
    float x[kRegGroup];
#pragma unroll
    for (int f = 0; f < kRegGroup; ++f) x[f] = f < cnt ? src[f0 + f] : 0.0f;
    float amax = 0.0f;
#pragma unroll
    for (int f = 0; f < kRegGroup; ++f) amax = fmaxf(amax, fabsf(x[f]));
    const float s = group_scale<BITS>(amax);
    *v_scales = s;
#pragma unroll
    for (int f = 0; f < kRegGroup; f += kStep) {
      if (f < g) {
        unsigned byte = f < cnt ? stored_code<BITS>(x[f], s) : kZero;
        if (BITS == 4) byte |= (f + 1 < cnt ? stored_code<BITS>(x[f + 1], s) : kZero) << 4;
        codes[v_code_byte(L, t, f0 + f)] = static_cast<uint8_t>(byte);
      }
    }
    return;
  }
  float amax = 0.0f;
  for (int f = 0; f < cnt; ++f) amax = fmaxf(amax, fabsf(src[f0 + f]));
  const float s = group_scale<BITS>(amax);
  *v_scales = s;
  auto code = [&](int f) -> unsigned { return f < cnt ? stored_code<BITS>(src[f0 + f], s) : kZero; };
  for (int f = 0; f < g; f += kStep) {
    const unsigned byte = BITS == 4 ? (code(f) | (code(f + 1) << 4)) : code(f);
    codes[v_code_byte(L, t, f0 + f)] = static_cast<uint8_t>(byte);
  }
}

// One-token append (a decode step), with each group spread over lanes: a
// lane holds one stored byte (two elements for 4-bit, one for 8-bit), the
// group's largest magnitude is a max over its kLanes = group / (elements per
// byte) neighbouring lanes (a power of two <= 64, so a group never straddles
// a wavefront), and every lane quantizes its own one or two elements.
// Threads [0, BH*D*kLanes): K, lane = token slot of the open group (fastest)
// and channel; the rest: V, lane = byte column of the new token's row.
// Same arithmetic as the general kernel (group_scale, stored_code), so the
// bytes are the same.
template <int BITS>
__global__ __launch_bounds__(256) void append_one_kernel(const float* __restrict__ k_new,
                                                         const float* __restrict__ v_new,
                                                         long long BH, Layout L, int N,
                                                         int lanes_log2,
                                                         uint8_t* __restrict__ k_codes,
                                                         float* __restrict__ k_scales,
                                                         uint8_t* __restrict__ v_codes,
                                                         float* __restrict__ v_scales,
                                                         float* __restrict__ k_tail) {
  constexpr int kStep = BITS == 4 ? 2 : 1;
  constexpr unsigned kZero = Codec<BITS>::kQmaxInt;
  const int lanes = 1 << lanes_log2;  // bytes (lanes) per group
  const long long tid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int D = L.D, g = L.group;
  const long long nk = BH * D * lanes;
  const bool k_part = tid < nk;
  const long long i = k_part ? tid : tid - nk;
  const int slot = static_cast<int>(i & (lanes - 1));
  const long long rest = i >> lanes_log2;
  float x[kStep];
  long long bh;
  int d = 0, t0 = 0, f0 = 0;
  bool live;
  if (k_part) {
    d = static_cast<int>(rest % D);
    bh = rest / D;
    const int g0 = N / g * g;  // the open group
    t0 = g0 + kStep * slot;
    live = true;
    const float* tail = k_tail + bh * g * static_cast<long long>(D) + d;
#pragma unroll
    for (int e = 0; e < kStep; ++e) {
      const int t = t0 + e;
      x[e] = t < N ? tail[static_cast<long long>(t - g0) * D]
                   : (t == N ? k_new[bh * D + d] : 0.0f);
    }
  } else {
    const int cols = L.dpad / kStep;  // byte columns of one token row
    f0 = kStep * static_cast<int>(rest % (cols >> lanes_log2) * lanes + slot);
    bh = rest / (cols >> lanes_log2);
    live = bh < BH;
#pragma unroll
    for (int e = 0; e < kStep; ++e)
      x[e] = live && f0 + e < D ? v_new[bh * D + f0 + e] : 0.0f;
  }
  float amax = fabsf(x[0]);
  if (BITS == 4) amax = fmaxf(amax, fabsf(x[kStep - 1]));
  for (int o = lanes >> 1; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (!live) return;
  const float s = group_scale<BITS>(amax);
  if (k_part) {
    const int g0 = N / g * g;
    if (slot == 0) k_scales[bh * k_scales_per_head(L) + k_scale_index(L, g0, d)] = s;
    if (t0 < L.nblocks * kBlockTokens) {
      unsigned byte = t0 <= N ? stored_code<BITS>(x[0], s) : kZero;
      if (BITS == 4) byte |= (t0 + 1 <= N ? stored_code<BITS>(x[1], s) : kZero) << 4;
      k_codes[bh * k_code_bytes_per_head(L) + k_code_byte(L, t0, d)] = static_cast<uint8_t>(byte);
    }
    // the new token joins the tail unless it completes its group
    if ((N + 1) % g != 0 && t0 <= N && N < t0 + kStep)
      k_tail[(bh * g + N % g) * static_cast<long long>(D) + d] = x[N - t0];
  } else {
    if (slot == 0) v_scales[bh * v_scales_per_head(L) + v_scale_index(L, N, f0)] = s;
    unsigned byte = f0 < D ? stored_code<BITS>(x[0], s) : kZero;
    if (BITS == 4) byte |= (f0 + 1 < D ? stored_code<BITS>(x[1], s) : kZero) << 4;
    v_codes[bh * v_code_bytes_per_head(L) + v_code_byte(L, N, f0)] = static_cast<uint8_t>(byte);
  }
}

// The new open group's tokens [n1 - n1 % g, n1) into the tail, one thread
// per (head, channel), after append_kernel has read the old tail.
__global__ __launch_bounds__(256) void append_tail_kernel(const float* __restrict__ k_new,
                                                          long long BH, int D, int N, int T,
                                                          int g, float* __restrict__ k_tail) {
  const long long tid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tid >= BH * D) return;
  const int d = static_cast<int>(tid % D);
  const long long bh = tid / D;
  const int n1 = N + T;
  for (int t = n1 / g * g; t < n1; ++t)
    k_tail[(bh * g + t % g) * D + d] = k_new[(bh * T + (t - N)) * D + d];
}

template <int BITS>
hipError_t pack_bits(const float* x, long long BH, const Layout& L, bool k_style, uint8_t* codes,
                     float* scales, hipStream_t stream) {
  if (L.D <= kStageMaxD) {
    const unsigned grid = static_cast<unsigned>(BH * L.nblocks);
    const size_t tile = sizeof(float) * kBlockTokens * (L.D + 1);
    if (!k_style) {
      const size_t lds = tile + sizeof(float) * L.vgroups * kBlockTokens;
      hipLaunchKernelGGL(pack_v_block_kernel<BITS>, dim3(grid), dim3(256), lds, stream, x, L,
                         scales, codes);
    } else if (kBlockTokens % L.group == 0) {
      const size_t lds = tile + sizeof(float) * (kBlockTokens / L.group) * L.D;
      hipLaunchKernelGGL((pack_k_block_kernel<BITS, true>), dim3(grid), dim3(256), lds, stream, x,
                         L, scales, codes);
    } else {
      hipLaunchKernelGGL(pack_k_scales_kernel<BITS>, dim3(grid_for(BH * L.kgroups * L.D)),
                         dim3(256), 0, stream, x, BH, L, scales);
      hipLaunchKernelGGL((pack_k_block_kernel<BITS, false>), dim3(grid), dim3(256), tile, stream,
                         x, L, scales, codes);
    }
    return hipGetLastError();
  }
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

hipError_t launch_cache_clear(int B, int H, int cap, int D, int bits, int group, uint8_t* k_codes,
                              float* k_scales, uint8_t* v_codes, float* v_scales,
                              hipStream_t stream) {
  const long long BH = static_cast<long long>(B) * H;
  const Layout L = make_layout(cap, D, bits, group);
  const uint8_t zero = bits == 4 ? 0x77 : 0x7F;  // stored code qmax (both nibbles for 4-bit)
  const long long most = BH * (k_code_bytes_per_head(L) > v_code_bytes_per_head(L)
                                   ? k_code_bytes_per_head(L)
                                   : v_code_bytes_per_head(L));
  const unsigned grid = most > 4096LL * 256 ? 4096u : grid_for(most);
  hipLaunchKernelGGL(cache_clear_kernel, dim3(grid), dim3(256), 0, stream, k_codes,
                     BH * k_code_bytes_per_head(L), k_scales, BH * k_scales_per_head(L), v_codes,
                     BH * v_code_bytes_per_head(L), v_scales, BH * v_scales_per_head(L), zero);
  return hipGetLastError();
}

hipError_t launch_append(const float* k_new, const float* v_new, int B, int H, int N, int T,
                         int cap, int D, int bits, int group, uint8_t* k_codes, float* k_scales,
                         uint8_t* v_codes, float* v_scales, float* k_tail, hipStream_t stream) {
  const long long BH = static_cast<long long>(B) * H;
  const Layout L = make_layout(cap, D, bits, group);
  const int per_byte = bits == 4 ? 2 : 1;
  const int lanes = group / per_byte;  // bytes per group
  if (T == 1 && lanes <= 64 && (lanes & (lanes - 1)) == 0) {
    int lanes_log2 = 0;
    while ((1 << lanes_log2) < lanes) ++lanes_log2;
    const long long threads = BH * D * lanes + BH * (L.dpad / per_byte);
    if (bits == 4)
      hipLaunchKernelGGL(append_one_kernel<4>, dim3(grid_for(threads)), dim3(256), 0, stream,
                         k_new, v_new, BH, L, N, lanes_log2, k_codes, k_scales, v_codes, v_scales,
                         k_tail);
    else
      hipLaunchKernelGGL(append_one_kernel<8>, dim3(grid_for(threads)), dim3(256), 0, stream,
                         k_new, v_new, BH, L, N, lanes_log2, k_codes, k_scales, v_codes, v_scales,
                         k_tail);
    return hipGetLastError();
  }
  const int n1 = N + T;
  const int ng = (n1 + group - 1) / group - N / group;  // token groups the new tokens touch
  // The tail is rewritten in the same launch unless the first touched group
  // reads it (N inside a group) while a later group is the new open one.
  const bool tail_here = ng == 1 || N % group == 0;
  const unsigned grid =
      grid_for(BH * ng * static_cast<long long>(D) + BH * T * static_cast<long long>(L.vgroups));
  if (bits == 4)
    hipLaunchKernelGGL(append_kernel<4>, dim3(grid), dim3(256), 0, stream, k_new, v_new, BH, L, N,
                       T, ng, tail_here, k_codes, k_scales, v_codes, v_scales, k_tail);
  else
    hipLaunchKernelGGL(append_kernel<8>, dim3(grid), dim3(256), 0, stream, k_new, v_new, BH, L, N,
                       T, ng, tail_here, k_codes, k_scales, v_codes, v_scales, k_tail);
  if (!tail_here && n1 % group != 0)
    hipLaunchKernelGGL(append_tail_kernel, dim3(grid_for(BH * D)), dim3(256), 0, stream, k_new, BH,
                       D, N, T, group, k_tail);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const float* scales, int B, int H, int N, int D,
                          int bits, int group, bool k_style, float* out, hipStream_t stream) {
  const long long BH = static_cast<long long>(B) * H;
  const Layout L = make_layout(N, D, bits, group);
  // heads over y (at most 65535) and z
  const unsigned hy = static_cast<unsigned>(BH < 65535 ? BH : 65535);
  const unsigned hz = static_cast<unsigned>((BH + hy - 1) / hy);
  const bool quad = D % 4 == 0 && reinterpret_cast<uintptr_t>(codes) % 4 == 0 &&
                    reinterpret_cast<uintptr_t>(scales) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(out) % 16 == 0;
  if (quad) {
    const dim3 g4(grid_for(static_cast<long long>(N) * (D / 4)), hy, hz);
    if (k_style) {
      if (bits == 4)
        hipLaunchKernelGGL((dequant4_kernel<4, true>), g4, dim3(256), 0, stream, codes, scales,
                           BH, L, out);
      else
        hipLaunchKernelGGL((dequant4_kernel<8, true>), g4, dim3(256), 0, stream, codes, scales,
                           BH, L, out);
    } else {
      if (bits == 4)
        hipLaunchKernelGGL((dequant4_kernel<4, false>), g4, dim3(256), 0, stream, codes, scales,
                           BH, L, out);
      else
        hipLaunchKernelGGL((dequant4_kernel<8, false>), g4, dim3(256), 0, stream, codes, scales,
                           BH, L, out);
    }
    return hipGetLastError();
  }
  const dim3 grid(grid_for(static_cast<long long>(N) * D), hy, hz);
  if (k_style) {
    if (bits == 4)
      hipLaunchKernelGGL((dequant_kernel<4, true>), grid, dim3(256), 0, stream, codes, scales, BH,
                         L, out);
    else
      hipLaunchKernelGGL((dequant_kernel<8, true>), grid, dim3(256), 0, stream, codes, scales, BH,
                         L, out);
  } else {
    if (bits == 4)
      hipLaunchKernelGGL((dequant_kernel<4, false>), grid, dim3(256), 0, stream, codes, scales,
                         BH, L, out);
    else
      hipLaunchKernelGGL((dequant_kernel<8, false>), grid, dim3(256), 0, stream, codes, scales,
                         BH, L, out);
  }
  return hipGetLastError();
}

}  // namespace kvq
