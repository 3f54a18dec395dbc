// General fused attention over the packed cache, plain float32 VALU
// arithmetic.  Serves every supported format (4/8-bit, any even group,
// D in {32, 64, 128}, up to 64 query rows per KV head) and the float32-cache
// path; the 4- and 8-bit group-32 D=128 cases have matrix-core kernels.
//
// Method, from "Block KV decoding: less workspace, more time"
// (huhohoo.com/en/docs/llm/kv-block-decode-cost), section "Do not average
// independently normalized blocks", and "给长前缀列一张有单位的资源账本"
// (codingai-lec05.pages.dev resource-ledger), section "why FlashAttention
// need not keep the whole heat map": per query row keep the running max m,
// the exponential sum z and the unnormalized value sum u; for each block
//   m' = max(m, max s),  a = 2^(m - m'),  z' = a z + sum 2^(s - m'),
//   u' = a u + sum 2^(s - m') v,
// and finally out = u / z.  Scores are in base-2 units (q is pre-multiplied
// by sm_scale * log2 e), which leaves the softmax unchanged.
//
// Work split: one workgroup per (KV split, KV head, batch).  A tile of
// kTile tokens is decoded to float32 in LDS (the exact value
// fl32((stored - qmax) * scale) the decode-all path produces), shared by
// all query rows of the KV head (every GQA head and query), then scored,
// folded into (m, z) and into u.  With several splits the last workgroup of
// a head to finish merges all of them (a ticket per head).
#include "kvq_internal.h"
#include "kvq_layout.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;

// Decoded K (token n, channel d) and V (token n, feature f) of head bh:
// fl32((stored - qmax) * scale), addressed through the block layout; the
// tokens of a recent-token window (n >= N - W) come from its float32 rows.
template <int SRC>
__device__ __forceinline__ float decode_k(const AttendProblem& p, const Layout& L, long long bh,
                                          int d, int n) {
  if (SRC == 32) return p.k_f32[(bh * p.N + n) * p.D + d];
  if (n >= p.N - p.W) return p.k_win[(bh * p.W + (n - (p.N - p.W))) * p.D + d];
  const unsigned b = p.k_codes[bh * k_code_bytes_per_head(L) + k_code_byte(L, n, d)];
  const int c = SRC == 4 ? static_cast<int>((n & 1) ? (b >> 4) : (b & 15u)) - 7
                         : static_cast<int>(b) - 127;
  return static_cast<float>(c) * p.k_scales[bh * k_scales_per_head(L) + k_scale_index(L, n, d)];
}

template <int SRC>
__device__ __forceinline__ float decode_v(const AttendProblem& p, const Layout& L, long long bh,
                                          int n, int f) {
  if (SRC == 32) return p.v_f32[(bh * p.N + n) * p.D + f];
  if (n >= p.N - p.W) return p.v_win[(bh * p.W + (n - (p.N - p.W))) * p.D + f];
  const unsigned b = p.v_codes[bh * v_code_bytes_per_head(L) + v_code_byte(L, n, f)];
  const int c = SRC == 4 ? static_cast<int>((f & 1) ? (b >> 4) : (b & 15u)) - 7
                         : static_cast<int>(b) - 127;
  return static_cast<float>(c) * p.v_scales[bh * v_scales_per_head(L) + v_scale_index(L, n, f)];
}

// Tokens of 32-token block blk (t0 = 32 blk) into sK / sV, reading the
// block's code bytes as 4-byte words (every thread decodes whole words: K,
// one channel quad of two token columns; V, one token quad of one byte
// column): the packed tokens below min(t_end, t_win) decoded, the tokens of
// a recent-token window [t_win, t_end) left alone (another loop writes
// them), every other token 0.  Same values as decode_k / decode_v:
// fl32((stored - qmax) * scale).
// ks_row[tl]: offset of token t0 + tl's K scale row ((t0 + tl) / group * D),
// fgrp[f]: value group of feature f < D (f / group); both precomputed in LDS
// so the decode does no integer division.
// Merge of one output (row, element e of the out / part_u arrays) over all
// splits: M = max_s m_s, Z = sum_s 2^(m_s - M) z_s, U = sum_s 2^(m_s - M)
// u_s, read with device-scope loads in batches of kBatch splits whose loads
// are all issued before use; splits that saw no legal token (m = -inf) are
// skipped and a row no split saw gets 0.
__device__ __forceinline__ float merge_splits(const AttendProblem& p, long long total_rows,
                                              long long row, long long e) {
  constexpr int kBatch = 8;
  float M = -INFINITY, Z = 0.0f, U = 0.0f;
  for (int s0 = 0; s0 < p.splits; s0 += kBatch) {
    float ms[kBatch], zs[kBatch], us[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const long long s = min(s0 + j, p.splits - 1);
      ms[j] = __hip_atomic_load(&p.part_m[s * total_rows + row], __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
      zs[j] = __hip_atomic_load(&p.part_z[s * total_rows + row], __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
      us[j] = __hip_atomic_load(&p.part_u[s * total_rows * p.D + e], __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j >= p.splits) ms[j] = -INFINITY;
    float mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) mb = fmaxf(mb, ms[j]);
    if (mb == -INFINITY) continue;
    const float a = exp2f(M - mb);  // 0 while nothing is merged yet
    Z *= a;
    U *= a;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (ms[j] == -INFINITY) continue;
      const float w = exp2f(ms[j] - mb);
      Z = fmaf(w, zs[j], Z);
      U = fmaf(w, us[j], U);
    }
    M = mb;
  }
  return Z > 0.0f ? U / Z : 0.0f;
}

// kStaged: the block's K scale rows and V scales were copied to LDS (kss,
// vss; ks_row then counts from the first staged row), else they are read
// from the cache arrays.  kFull: every token of the block is packed and
// attended (no window token, none past the split), so no token is tested.
template <int D, int SRC, bool kStaged, bool kFull>
__device__ __forceinline__ void decode_block(const AttendProblem& p, const Layout& L, long long bh,
                                             int blk, int t_end, int t_win, float (*sK)[D + 1],
                                             float (*sV)[D], const int* ks_row,
                                             const int* fgrp, const float* kss,
                                             const float* vss) {
  constexpr int kQmax = SRC == 4 ? 7 : 127;
  constexpr int kKcols = kTile * SRC / 8;  // K byte columns per channel octet
  const int t0 = blk * kTile;
  const int t_pk = min(t_end, t_win);
  auto window = [&](int tl) { return !kFull && t0 + tl >= t_win && t0 + tl < t_end; };
  auto packed = [&](int tl) { return kFull || t0 + tl < t_pk; };
  const int tid = threadIdx.x;
  const unsigned* kw = reinterpret_cast<const unsigned*>(
      p.k_codes + bh * k_code_bytes_per_head(L) + static_cast<long long>(blk) * L.kblock_bytes);
  const float* ks = kStaged ? kss : p.k_scales + bh * k_scales_per_head(L);
  for (int w = tid; w < L.kblock_bytes / 4; w += kThreads) {
    const unsigned word = kw[w];
    const int run = w >> 1;  // 8-byte run (octet o, column j)
    const int o = run / kKcols, j = run % kKcols;
    const int d0 = 8 * o + 4 * (w & 1);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int d = d0 + b;
      if (d >= D) break;
      const unsigned byte = (word >> (8 * b)) & 255u;
      if (SRC == 4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int tl = 2 * j + h;
          if (window(tl)) continue;
          const int c = static_cast<int>(h ? byte >> 4 : byte & 15u) - kQmax;
          sK[tl][d] = packed(tl) ? static_cast<float>(c) * ks[ks_row[tl] + d] : 0.0f;
        }
      } else {
        if (window(j)) continue;
        const int c = static_cast<int>(byte) - kQmax;
        sK[j][d] = packed(j) ? static_cast<float>(c) * ks[ks_row[j] + d] : 0.0f;
      }
    }
  }
  const unsigned* vw = reinterpret_cast<const unsigned*>(
      p.v_codes + bh * v_code_bytes_per_head(L) + static_cast<long long>(blk) * L.vblock_bytes);
  const float* vs = kStaged ? vss
                           : p.v_scales + bh * v_scales_per_head(L) +
                                 static_cast<long long>(blk) * L.vgroups * kTile;  // [group][32 tokens]
  for (int w = tid; w < L.vblock_bytes / 4; w += kThreads) {
    const unsigned word = vw[w];
    const int run = w >> 1;  // 8-byte run (token octet o < 4, column f)
    const int o = (run >= L.vcols) + (run >= 2 * L.vcols) + (run >= 3 * L.vcols);
    const int col = run - o * L.vcols;
    const int tq = 8 * o + 4 * (w & 1);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int tl = tq + b;
      if (window(tl)) continue;
      const bool live = packed(tl);
      const unsigned byte = (word >> (8 * b)) & 255u;
      if (SRC == 4) {
        const int f = 2 * col;
        if (f >= D) continue;
        const float s = live ? vs[fgrp[f] * kTile + tl] : 0.0f;
        sV[tl][f] = live ? static_cast<float>(static_cast<int>(byte & 15u) - kQmax) * s : 0.0f;
        if (f + 1 < D)
          sV[tl][f + 1] = live ? static_cast<float>(static_cast<int>(byte >> 4) - kQmax) * s : 0.0f;
      } else {
        if (col >= D) continue;
        sV[tl][col] = live ? static_cast<float>(static_cast<int>(byte) - kQmax) *
                                 vs[fgrp[col] * kTile + tl]
                           : 0.0f;
      }
    }
  }
}

template <int D, int SRC>
__global__ __launch_bounds__(kThreads) void attend_valu_kernel(AttendProblem p) {
  constexpr int kAcc = kMaxRows * D / kThreads;  // u accumulators per thread
  __shared__ float sQ[kMaxRows][D + 1];  // padded: rows read together sit on distinct banks
  __shared__ float sK[kTile][D + 1];
  __shared__ __align__(16) float sV[kTile][D];
  __shared__ float sP[kMaxRows][kTile + 1];
  __shared__ float sM[kMaxRows], sZ[kMaxRows], sA[kMaxRows];
  __shared__ int sKsRow[kTile];     // K scale row offset of each token of the tile
  __shared__ int sLast;             // this workgroup is the last split of its head to finish
  __shared__ int sFgrp[D];          // value group of each feature below D
  // Groups of at least kStageMinGroup: a block's K scales span at most
  // kStageKRows rows and its V scales at most kStageVGroups groups; they are
  // copied to LDS once per tile (two contiguous runs) instead of being read
  // per decoded element.
  constexpr int kStageMinGroup = 8;
  constexpr int kStageKRows = 5;
  constexpr int kStageVGroups = (D + kStageMinGroup - 1) / kStageMinGroup;
  __shared__ float sKss[kStageKRows * D];
  __shared__ float sVss[kStageVGroups * kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int split = blockIdx.x;
  const int rows = p.rows;
  const long long bh = static_cast<long long>(blockIdx.z) * p.Hkv + blockIdx.y;
  const int t_begin = split * p.tokens_per_split;
  const int t_end = min(p.N, t_begin + p.tokens_per_split);
  const Layout L = make_layout(p.cap, p.D, SRC == 32 ? 8 : SRC, SRC == 32 ? 2 : p.group);

  // Query rows of this KV head are contiguous in q: [bh*rows, bh*rows + rows).
  for (int i = tid; i < rows * D; i += kThreads)
    sQ[i / D][i % D] = p.q[bh * rows * D + i] * p.qscale;
  for (int r = tid; r < rows; r += kThreads) {
    sM[r] = -INFINITY;
    sZ[r] = 0.0f;
  }
  if (SRC != 32)
    for (int f = tid; f < D; f += kThreads) sFgrp[f] = f / p.group;
  float acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i) acc[i] = 0.0f;
  // float32 cache with both arrays 16-byte aligned: vector row loads
  const bool f32_vec = SRC == 32 && ((reinterpret_cast<uintptr_t>(p.k_f32) |
                                      reinterpret_cast<uintptr_t>(p.v_f32)) & 15) == 0;
  __syncthreads();

  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    const int tn = min(kTile, t_end - t0);
    const int t_win = p.N - p.W;  // first token of a recent-token window (N without one)
    if (SRC != 32 && p.codes_aligned && t0 < t_win) {
      // Tiles start on block boundaries: decode the packed block word by
      // word, then the window's float32 rows of the tile (disjoint tokens).
      const bool staged = p.group >= kStageMinGroup;  // uniform
      if (staged) {
        const int row0 = t0 / p.group;
        const int row1 = min((t0 + kTile - 1) / p.group, L.kgroups - 1);
        const float* kr = p.k_scales + bh * k_scales_per_head(L) + static_cast<long long>(row0) * D;
        for (int i = tid; i < (row1 - row0 + 1) * D; i += kThreads) sKss[i] = kr[i];
        const float* vr = p.v_scales + bh * v_scales_per_head(L) +
                          static_cast<long long>(t0 / kTile) * L.vgroups * kTile;
        for (int i = tid; i < L.vgroups * kTile; i += kThreads) sVss[i] = vr[i];
        if (tid < kTile) sKsRow[tid] = (min((t0 + tid) / p.group, row1) - row0) * D;
      } else if (tid < kTile) {
        sKsRow[tid] = (t0 + tid) / p.group * D;
      }
      __syncthreads();
      const bool full = t0 + kTile <= min(t_end, t_win);  // uniform
      if (staged && full)
        decode_block<D, SRC, true, true>(p, L, bh, t0 / kTile, t_end, t_win, sK, sV, sKsRow,
                                         sFgrp, sKss, sVss);
      else if (staged)
        decode_block<D, SRC, true, false>(p, L, bh, t0 / kTile, t_end, t_win, sK, sV, sKsRow,
                                          sFgrp, sKss, sVss);
      else
        decode_block<D, SRC, false, false>(p, L, bh, t0 / kTile, t_end, t_win, sK, sV, sKsRow,
                                           sFgrp, nullptr, nullptr);
      if (t0 + kTile > t_win) {
        for (int i = tid; i < kTile * D; i += kThreads) {
          const int j = i / D, d = i % D;
          if (t0 + j >= t_win && j < tn) {
            sK[j][d] = decode_k<SRC>(p, L, bh, d, t0 + j);
            sV[j][d] = decode_v<SRC>(p, L, bh, t0 + j, d);
          }
        }
      }
    } else if (SRC == 32 && f32_vec) {
      // Float32 cache rows, 16-byte aligned: whole rows with 16-byte loads.
      const float* krow = p.k_f32 + (bh * p.N + t0) * D;
      const float* vrow = p.v_f32 + (bh * p.N + t0) * D;
      for (int i = tid; i < kTile * (D / 4); i += kThreads) {
        const int j = i / (D / 4), d = (i % (D / 4)) * 4;
        float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
        if (j < tn) {
          kk = *reinterpret_cast<const float4*>(krow + j * D + d);
          vv = *reinterpret_cast<const float4*>(vrow + j * D + d);
        }
        sK[j][d] = kk.x;
        sK[j][d + 1] = kk.y;
        sK[j][d + 2] = kk.z;
        sK[j][d + 3] = kk.w;
        *reinterpret_cast<float4*>(&sV[j][d]) = vv;
      }
    } else {
      // Element by element.  K: the 8 channels of an octet fastest, then the
      // token (one 8-byte run of the block layout per token column); V: the
      // feature fastest.
      for (int i = tid; i < kTile * D; i += kThreads) {
        const int j = (i >> 3) % kTile, d = (i / (8 * kTile)) * 8 + (i & 7);
        sK[j][d] = j < tn ? decode_k<SRC>(p, L, bh, d, t0 + j) : 0.0f;
      }
      for (int i = tid; i < kTile * D; i += kThreads) {
        const int f = i % D, j = i / D;
        sV[j][f] = j < tn ? decode_v<SRC>(p, L, bh, t0 + j, f) : 0.0f;
      }
    }
    __syncthreads();

    // Scores of every (row, token); tokens past N are masked out (-inf), and
    // in a causal chunk so are the tokens after the row's query position
    // (row r is query r % R of its head, at position N - R + r % R).
    for (int i = tid; i < rows * kTile; i += kThreads) {
      const int r = i / kTile, j = i % kTile;
      float s = -INFINITY;
      if (j < tn && (!p.causal || t0 + j <= p.pos_end - p.R + r % p.R)) {
        // four independent partial sums (no single dependent chain of D FMAs)
        float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
        for (int d = 0; d < D; d += 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) s4[e] = fmaf(sQ[r][d + e], sK[j][d + e], s4[e]);
        }
        s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      }
      sP[r][j] = s;
    }
    __syncthreads();

    // (m, z) update: each wave takes two rows at a time, one per 32-lane half.
    for (int rb = wave * 2; rb < rows; rb += 2 * (kThreads / 64)) {
      const int r = rb + (lane >> 5);
      const int j = lane & 31;
      const bool live = r < rows;
      const float s = live ? sP[r][j] : -INFINITY;
      float mx = s;
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float m_old = live ? sM[r] : 0.0f;
      // Without a causal mask the tile holds a real token for every row, so
      // m_new is finite.  A causal row that has seen no legal key yet keeps
      // m = -inf (and z = u = 0): its exponents are taken against 0 so that
      // (-inf) - (-inf) is never formed.
      const float m_new = fmaxf(m_old, mx);
      const float m_ref = m_new == -INFINITY ? 0.0f : m_new;
      const float pj = exp2f(s - m_ref);
      const float alpha = exp2f(m_old - m_ref);
      float sum = pj;
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
      if (live) {
        sP[r][j] = pj;
        if (j == 0) {
          sM[r] = m_new;
          sZ[r] = alpha * sZ[r] + sum;
          sA[r] = alpha;
        }
      }
    }
    __syncthreads();

    // u update: thread owns (row, feature) pairs; both z (above) and u
    // (here) are rescaled by the same alpha.
#pragma unroll
    for (int i = 0; i < kAcc; ++i) {
      // Slots past rows * D hold nothing for any thread: leave the loop (a
      // uniform exit, so the unrolled slots of the few-row case cost nothing).
      if (i * kThreads >= rows * D) break;
      const int idx = tid + i * kThreads;
      if (idx < rows * D) {
        const int r = idx / D, f = idx % D;
        float a2[2] = {0.0f, 0.0f};
#pragma unroll 8
        for (int j = 0; j < kTile; j += 2) {
          a2[0] = fmaf(sP[r][j], sV[j][f], a2[0]);
          a2[1] = fmaf(sP[r][j + 1], sV[j + 1][f], a2[1]);
        }
        const float add = a2[0] + a2[1];
        acc[i] = fmaf(sA[r], acc[i], add);
      }
    }
    __syncthreads();
  }

  const long long row0 = bh * rows;
  if (p.splits == 1) {
#pragma unroll
    for (int i = 0; i < kAcc; ++i) {
      const int idx = tid + i * kThreads;
      if (idx < rows * D) {
        const int r = idx / D;
        // z = 0 only for a causal row with no legal key: its output is 0.
        p.out[(row0 + r) * D + idx % D] = sZ[r] > 0.0f ? acc[i] / sZ[r] : 0.0f;
      }
    }
    return;
  }
  // Several splits: store this split's partial (m, z, u) with device-scope
  // stores, wait until they are acknowledged, take a ticket from the head's
  // arrival counter; the last split to arrive merges them all ([RL] "two
  // stops of the online accumulation") and resets the counter.
  const long long total_rows = static_cast<long long>(p.B) * p.Hkv * rows;
  const long long base = static_cast<long long>(split) * total_rows + row0;
#pragma unroll
  for (int i = 0; i < kAcc; ++i) {
    if (i * kThreads >= rows * D) break;
    const int idx = tid + i * kThreads;
    if (idx < rows * D)
      __hip_atomic_store(&p.part_u[base * D + idx], acc[i], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int r = tid; r < rows; r += kThreads) {
    __hip_atomic_store(&p.part_m[base + r], sM[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p.part_z[base + r], sZ[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores above are acknowledged
  __syncthreads();
  unsigned* counter = &p.counters[bh * kCounterStride];
  if (tid == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sLast = ticket_outcome(prev, p.splits);
  }
  __syncthreads();
  if (sLast == kTicketWait) return;
  if (sLast == kTicketStale) {  // the counter was not zero at the start: make it visible
#pragma unroll
    for (int i = 0; i < kAcc; ++i) {
      if (i * kThreads >= rows * D) break;
      const int idx = tid + i * kThreads;
      if (idx < rows * D)  // a quiet NaN, stored as its bit pattern
        reinterpret_cast<unsigned*>(p.out)[row0 * D + idx] = 0x7fc00000u;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kAcc; ++i) {
    if (i * kThreads >= rows * D) break;
    const int idx = tid + i * kThreads;
    if (idx < rows * D) p.out[row0 * D + idx] = merge_splits(p, total_rows, row0 + idx / D, row0 * D + idx);
  }
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D>
hipError_t launch_valu_d(const AttendProblem& p, hipStream_t stream) {
  const dim3 grid(p.splits, p.Hkv, p.B);
  switch (p.bits) {
    case 4: hipLaunchKernelGGL((attend_valu_kernel<D, 4>), grid, dim3(kThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((attend_valu_kernel<D, 8>), grid, dim3(kThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL((attend_valu_kernel<D, 32>), grid, dim3(kThreads), 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_valu(const AttendProblem& p, hipStream_t stream) {
  hipError_t e;
  switch (p.D) {
    case 32: e = launch_valu_d<32>(p, stream); break;
    case 64: e = launch_valu_d<64>(p, stream); break;
    default: e = launch_valu_d<128>(p, stream); break;
  }
  return e;
}

}  // namespace kvq
