// Byte layout of the packed cache in device memory.
//
// The quantization itself follows "KV分组打包：4-bit到底省了多少？"
// (huhohoo.com/docs/llm/kv-packed-groups), "what a byte holds" and "why
// grouping needs both direction and length": K is grouped along tokens
// inside a channel, V along features inside a token, one float32 scale per
// group, and a 4-bit byte holds two neighbouring codes of one group, the
// lower-indexed one in the low nibble.  The pages fix the groups and the
// byte contents, not the order of the bytes; this file fixes that order,
// chosen so that the attention kernels read whole 32-token blocks with
// contiguous, fully coalesced loads that land in the registers in the
// order the matrix cores consume them.
//
// Per (batch, head) the cache is cut into blocks of 32 tokens
// (nblocks = ceil(N / 32)); every position that holds no quantized element
// (tokens past N, channels past D, features past the last group) stores the
// zero code (7 for 4-bit, 127 for 8-bit).
//
//   K codes : [B][H][nblocks][kblock_bytes]; inside a block, byte
//             (o, j, e) at (o * kcols + j) * 8 + e holds channel d = 8 o + e
//             of byte column j, o < ceil(D / 8), kcols = 32 * bits / 8.
//             4-bit column j = tokens 2j (low nibble) and 2j + 1 (high);
//             8-bit column j = token j.
//   K scales: [B][H][ceil(N / group)][D]   (group-major: the scales of one
//             token group are contiguous over channels).
//   V codes : [B][H][nblocks][vblock_bytes]; inside a block, byte
//             (o, f, e) at (o * vcols + f) * 8 + e holds token 8 o + e
//             (o < 4) of byte column f, vcols = Dpad * bits / 8 with
//             Dpad = D rounded up to the group.  4-bit column f = features
//             2f (low nibble) and 2f + 1 (high); 8-bit column f = feature f.
//   V scales: [B][H][nblocks][Dpad / group][32]  (token-minor; tokens past
//             N carry scale 1, the scale of an all-zero group).
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {

constexpr int kBlockTokens = 32;

struct Layout {
  int N, D, bits, group;
  int nblocks;            // ceil(N / 32)
  int d8;                 // ceil(D / 8): K channel octets
  int kcols;              // K byte columns per block: 32 * bits / 8
  long long kblock_bytes; // d8 * kcols * 8
  int kgroups;            // ceil(N / group): K scale rows
  int dpad;               // D rounded up to the group
  int vcols;              // V byte columns per token octet: dpad * bits / 8
  long long vblock_bytes; // 4 * vcols * 8
  int vgroups;            // dpad / group
};

__host__ __device__ inline Layout make_layout(int N, int D, int bits, int group) {
  Layout L;
  L.N = N;
  L.D = D;
  L.bits = bits;
  L.group = group;
  L.nblocks = (N + kBlockTokens - 1) / kBlockTokens;
  L.d8 = (D + 7) / 8;
  L.kcols = kBlockTokens * bits / 8;
  L.kblock_bytes = static_cast<long long>(L.d8) * L.kcols * 8;
  L.kgroups = (N + group - 1) / group;
  L.dpad = (D + group - 1) / group * group;
  L.vcols = L.dpad * bits / 8;
  L.vblock_bytes = 4LL * L.vcols * 8;
  L.vgroups = L.dpad / group;
  return L;
}

// Per-head element counts.
__host__ __device__ inline long long k_code_bytes_per_head(const Layout& L) {
  return L.nblocks * L.kblock_bytes;
}
__host__ __device__ inline long long k_scales_per_head(const Layout& L) {
  return static_cast<long long>(L.kgroups) * L.D;
}
__host__ __device__ inline long long v_code_bytes_per_head(const Layout& L) {
  return L.nblocks * L.vblock_bytes;
}
__host__ __device__ inline long long v_scales_per_head(const Layout& L) {
  return static_cast<long long>(L.nblocks) * L.vgroups * kBlockTokens;
}

// Byte (within one head) holding K element (token t, channel d); for 4-bit
// codes the element is the high nibble when t is odd.
__host__ __device__ inline long long k_code_byte(const Layout& L, int t, int d) {
  const int blk = t / kBlockTokens, tl = t % kBlockTokens;
  const int j = L.bits == 4 ? tl >> 1 : tl;
  return blk * L.kblock_bytes + (static_cast<long long>(d >> 3) * L.kcols + j) * 8 + (d & 7);
}

// Byte (within one head) holding V element (token t, feature f); for 4-bit
// codes the element is the high nibble when f is odd.
__host__ __device__ inline long long v_code_byte(const Layout& L, int t, int f) {
  const int blk = t / kBlockTokens, tl = t % kBlockTokens;
  const int col = L.bits == 4 ? f >> 1 : f;
  return blk * L.vblock_bytes + (static_cast<long long>(tl >> 3) * L.vcols + col) * 8 + (tl & 7);
}

__host__ __device__ inline long long k_scale_index(const Layout& L, int t, int d) {
  return static_cast<long long>(t / L.group) * L.D + d;
}

__host__ __device__ inline long long v_scale_index(const Layout& L, int t, int f) {
  return (static_cast<long long>(t / kBlockTokens) * L.vgroups + f / L.group) * kBlockTokens +
         t % kBlockTokens;
}

}  // namespace kvq
