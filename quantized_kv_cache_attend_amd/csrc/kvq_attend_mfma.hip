// Matrix-core fused attention for the 4-bit, group-32, D=128 packed cache
// with at most 4 query rows per KV head (GQA group x queries <= 4).
//
// Method: the blocked online softmax of "Block KV decoding: less workspace,
// more time" (huhohoo.com/en/docs/llm/kv-block-decode-cost), section "Do not
// average independently normalized blocks", and of "给长前缀列一张有单位的资源账本"
// (codingai-lec05.pages.dev resource-ledger), section "why FlashAttention need
// not keep the whole heat map": per query row a running max m, exponential
// sum z and unnormalized value sum u, with z and u both rescaled by
// 2^(m_old - m_new) whenever a 32-token block raises the max.  Scores are in
// base-2 units (q carries sm_scale * log2 e).  KV splits (and the four waves
// of a workgroup) are merged with the same rescale ("two stops of the online
// accumulation" on the same page: partial statistics are composable).
//
// Packed format ("KV分组打包：4-bit到底省了多少？", huhohoo.com/docs/llm/kv-packed-groups,
// "what a byte holds", "why grouping needs both direction and length"):
// K codes are channel-major, [d][token pairs], one float32 scale per
// (channel, 32-token group); V codes are token-major, [token][feature
// pairs], one scale per (token, 32-feature group); value = (stored - 7) * s.
//
// Exact code operands.  Each stored nibble c is turned into the fp16 value
// c - 7 exactly: OR-ing it into the mantissa of 0x6400 gives 1024 + c (low
// nibble) or 1024 + 16c (high nibble, masked in place), and one packed fp16
// add (or multiply-add by 1/16) removes the bias.  All matrix-core operands
// stay in the fp16 normal range: products with fp16 subnormal operands were
// measured to lose low bits when accumulated onto a larger accumulator.
//
// Float32 factors on fp16 matrix cores.  q~[r][d] = q[r][d] * qscale *
// sK[d][G] (scores) and p~[r][j] = p[r][j] * sV[j][G'] (values) are split
// into fp16 hi + lo (round toward zero, then the remainder), so each product
// carries ~22 significant bits and accumulates in float32.  Before the split
// each set is multiplied by a power of two 2^S that puts its largest element
// in [2^14, 2^15) (per 32-channel group and query row for q~, per tile and
// value group for the V scales); the factor is exact and is divided out in
// float32 afterwards.  It keeps the lo halves of all but negligible elements
// out of the fp16 subnormal range.
//
// Tiling.  A workgroup (4 waves) owns one KV head and a run of 256-token
// tiles.  Per tile the whole workgroup streams K codes (128 channels x 128
// bytes), V codes (256 tokens x 64 bytes) and both scale sets into LDS with
// coalesced 16-byte loads, precomputes q~ for the tile's 8 groups (shared by
// all query rows), then each wave takes two 32-token chunks:
//   S^T[token][col] = codes^T (A: 16 token pairs x 32 channels, from LDS by
//     ds_read_b64_tr_b8, which hands each lane 8 channels of one token pair)
//     x q~^T (B: 32 channels x 16 columns; column n = (hi|lo, row n % 4));
//   u[4 G' + r][f] += p~_G'(A: 16 rows = 4 value groups x 4 query rows)
//     x V codes (B: 32 tokens x 16 feature pairs, again by tr_b8).
// The A-row layout 4*G' + r lets every lane compute the p~ of one value
// group only; the rows whose group differs from the B columns' group are
// discarded.  With at most 4 query rows the matrix cores are far from busy,
// so spending MFMA issue to save VALU work is the right trade.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kD = 128;
constexpr int kTile = 256;              // tokens per workgroup tile
constexpr int kChunks = kTile / 32;     // 32-token chunks (= K groups) per tile
constexpr int kKRow = 144;              // LDS bytes per K channel row: 128 + 16 pad
constexpr int kVRow = 80;               // LDS bytes per V token row: 64 + 16 pad
// s_waitcnt immediate for vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt left at max)
constexpr unsigned kWaitVmcnt0 = 0x0F70;

struct alignas(16) Smem {
  union {
    struct {
      uint8_t k[kD * kKRow];                    // K codes, [channel][tile bytes]
      uint8_t v[kTile * kVRow];                 // V codes, [token][feature-pair bytes]
    } codes;
    float wu[kWaves][4][kD];                    // per-wave u, for the wave merge
  } big;
  _Float16 qt[kChunks][4][2][4][4][8];          // q~ [group][kstep][hi|lo][row][kblock][8]
  float vs[kChunks][4][4][8];                   // V scales [chunk][token octet][group][8]
  float ks[kChunks][kD];                        // K scales [group][channel]
  float qunscale[kChunks][4];                   // 2^-S per [group][row]
  float vmax[kWaves];                           // per-wave max V scale of the tile
  float wm[kWaves][4];
  float wz[kWaves][4];
  int last;
};

__device__ __forceinline__ unsigned as_u32(float x) { return __builtin_bit_cast(unsigned, x); }
__device__ __forceinline__ float as_f32(unsigned x) { return __builtin_bit_cast(float, x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// S with max_abs * 2^S in [2^14, 2^15) (0 for a zero maximum), clamped so the
// scaled values and the inverse factors stay finite and normal in float32.
__device__ __forceinline__ int prescale_exp(float max_abs) {
  if (!(max_abs > 0.0f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(max_abs);
  return min(100, max(-100, 15 - e));
}

// value of lane (n + 8) % 16 within each 16-lane row
__device__ __forceinline__ float row_ror8(float x) {
  return as_f32(static_cast<unsigned>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(as_u32(x)), 0x128, 0xf, 0xf, false)));
}
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return as_f32(static_cast<unsigned>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(as_u32(x)), kCtrl, 0xf, 0xf, false)));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124;

// Max / sum over one query row.  Lane (n, q) holds row n % 4 for the eight
// tokens 8q..8q+7 of a chunk; lanes with equal n % 4 and equal q hold
// identical copies, so only the four 16-lane q-blocks are reduced, with the
// gfx950 row-swap instructions (lane ^ 16, lane ^ 32) instead of LDS
// permutes.
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  a = as_f32(r[0]);
  b = as_f32(r[1]);
}
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  a = as_f32(r[0]);
  b = as_f32(r[1]);
}
__device__ __forceinline__ float row_max(float x) {
  float a, b;
  swap16(x, a, b);
  x = fmaxf(a, b);
  swap32(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float row_sum(float x) {
  float a, b;
  swap16(x, a, b);
  x = a + b;
  swap32(x, a, b);
  return a + b;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Constants kept in VGPRs: gfx9 VOP3 encodings take no literal operand and
// at most one scalar one, so this lets each nibble extraction be a single
// v_and_or_b32.
struct CodeConsts {
  unsigned lo_mask, hi_mask, magic;
};
__device__ __forceinline__ unsigned in_vgpr(unsigned x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ CodeConsts code_consts() {
  return {in_vgpr(0x000F000Fu), in_vgpr(0x00F000F0u), in_vgpr(0x64006400u)};
}

// Eight code bytes b0..b7 (from one transposed LDS read) -> fp16 (c - 7) of
// their low nibbles (lo) and high nibbles (hi), in k-slot order
// (b0, b2, b1, b3, b4, b6, b5, b7).  OR-ing a nibble into 0x6400 gives
// 1024 + c (low) or 1024 + 16c (high, masked in place); one packed add, or
// multiply-add by 1/16, removes the bias exactly.
__device__ __forceinline__ void codes_to_half(i32x2 w, const CodeConsts& k, half8_t& lo,
                                              half8_t& hi) {
  const half2_t bias_lo = {(_Float16)-1031.0f, (_Float16)-1031.0f};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t bias_hi = {(_Float16)-71.0f, (_Float16)-71.0f};
  const unsigned src[4] = {static_cast<unsigned>(w.x), static_cast<unsigned>(w.x) >> 8,
                           static_cast<unsigned>(w.y), static_cast<unsigned>(w.y) >> 8};
  u32x4 l, h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned xl = (src[i] & k.lo_mask) | k.magic;
    const unsigned xh = (src[i] & k.hi_mask) | k.magic;
    l[i] = __builtin_bit_cast(unsigned, __builtin_bit_cast(half2_t, xl) + bias_lo);
    h[i] = __builtin_bit_cast(
        unsigned, __builtin_elementwise_fma(__builtin_bit_cast(half2_t, xh), sixteenth, bias_hi));
  }
  lo = __builtin_bit_cast(half8_t, l);
  hi = __builtin_bit_cast(half8_t, h);
}

// k-slot j of a converted operand holds byte kSlotByte[j] of the 8 read.
__device__ constexpr int kSlotByte[8] = {0, 2, 1, 3, 4, 6, 5, 7};

__device__ __forceinline__ i32x2 lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
}

__device__ __forceinline__ f32x4 mfma(half8_t a, half8_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp16 hi/lo split of 8 float32 values, packed in k-slot order.
__device__ __forceinline__ void split_hilo(const float x[8], half8_t& hi, half8_t& lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    auto hp = __builtin_amdgcn_cvt_pkrtz(x[2 * i], x[2 * i + 1]);
    const float r0 = x[2 * i] - static_cast<float>(hp[0]);
    const float r1 = x[2 * i + 1] - static_cast<float>(hp[1]);
    auto lp = __builtin_amdgcn_cvt_pkrtz(r0, r1);
    h[i] = __builtin_bit_cast(unsigned, hp);
    l[i] = __builtin_bit_cast(unsigned, lp);
  }
  hi = __builtin_bit_cast(half8_t, h);
  lo = __builtin_bit_cast(half8_t, l);
}


// Per-thread registers of one staged tile (filled by load_tile, consumed by
// stage_tile); two of them form the prefetch double buffer.
struct TileRegs {
  u32x4 k[4];   // K codes: (channel idx>>3, 16-byte segment idx&7), idx = tid + 256 i
  u32x4 v[4];   // V codes: (token idx>>2, 16-byte segment idx&3)
  f32x4 sk;     // K scales of channel tid&127, groups 4*(tid>>7) .. +3 of the tile
  u32x4 sv;     // V scales of token tid (4 value groups)
};

struct Head {
  const uint8_t* kc;
  const float* ksc;
  const uint8_t* vc;
  const float* vsc;
  int N, npad, ngroups;
  long long krow_bytes;
};

// Issue every global load of one 256-token tile.  Interior tiles take the
// plain path; the last tile of the cache reads clamped in-range addresses
// and zero-fills what lies past the padded K row or past token N, so no
// load sits behind a branch and all of them are in flight together.
__device__ __forceinline__ void load_tile(const Head& h, int tile0, int tid, TileRegs& r) {
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const int d = tid & 127, gh = (tid >> 7) * 4;
  if (tile0 + kTile <= h.N) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kThreads * i;
      r.k[i] = *reinterpret_cast<const u32x4*>(h.kc + (idx >> 3) * h.krow_bytes + (tile0 >> 1) +
                                               (idx & 7) * 16);
      r.v[i] = *reinterpret_cast<const u32x4*>(
          h.vc + static_cast<long long>(tile0 + (idx >> 2)) * 64 + (idx & 3) * 16);
    }
    const float* ks = h.ksc + static_cast<long long>(d) * h.ngroups + (tile0 >> 5) + gh;
    if ((h.ngroups & 3) == 0) {
      r.sk = *reinterpret_cast<const f32x4*>(ks);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) r.sk[i] = ks[i];
    }
    r.sv = *reinterpret_cast<const u32x4*>(h.vsc + static_cast<long long>(tile0 + tid) * 4);
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + kThreads * i;
    const int s = idx & 7;
    const bool kin = tile0 + s * 32 < h.npad;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(
        h.kc + (idx >> 3) * h.krow_bytes + (kin ? (tile0 >> 1) + s * 16 : 0));
    r.k[i] = kin ? kv : zero4;
    const int j = idx >> 2;
    const bool vin = tile0 + j < h.N;
    const u32x4 vv = *reinterpret_cast<const u32x4*>(
        h.vc + static_cast<long long>(vin ? tile0 + j : 0) * 64 + (idx & 3) * 16);
    r.v[i] = vin ? vv : zero4;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = (tile0 >> 5) + gh + i;
    const float v = h.ksc[static_cast<long long>(d) * h.ngroups + (g < h.ngroups ? g : 0)];
    r.sk[i] = g < h.ngroups ? v : 0.0f;
  }
  const bool vin = tile0 + tid < h.N;
  const u32x4 sv =
      *reinterpret_cast<const u32x4*>(h.vsc + static_cast<long long>(vin ? tile0 + tid : 0) * 4);
  r.sv = vin ? sv : zero4;
}

// Running softmax state of one wave.  Lane (n, q) tracks query row n % 4;
// acc[g][e] holds the value sums of feature group g, even (e = 0) or odd
// (e = 1) features, rows 4q + i = (value group q, query row i), in units of
// 2^sv.
struct WaveState {
  float m_run, z_run;
  f32x4 acc[4][2];
  bool live;  // a block has been folded in (acc may be non-zero)
};

__device__ __forceinline__ void scale_acc(WaveState& st, f32x4 f) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    st.acc[g][0] *= f;
    st.acc[g][1] *= f;
  }
}

// Write one tile's registers to LDS (codes, K scales, raw V scales) and
// each wave's maximum V scale.  The registers are free again afterwards.
__device__ __forceinline__ void stage_tile(Smem& sm, const TileRegs& r) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + kThreads * i;
    *reinterpret_cast<u32x4*>(&sm.big.codes.k[(idx >> 3) * kKRow + (idx & 7) * 16]) = r.k[i];
    *reinterpret_cast<u32x4*>(&sm.big.codes.v[(idx >> 2) * kVRow + (idx & 3) * 16]) = r.v[i];
  }
  {
    const int d = tid & 127, gh = (tid >> 7) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.ks[gh + i][d] = r.sk[i];
    float vmx = fmaxf(fmaxf(as_f32(r.sv[0]), as_f32(r.sv[1])),
                      fmaxf(as_f32(r.sv[2]), as_f32(r.sv[3])));
    vmx = fmaxf(vmx, dpp<kRowRor1>(vmx));
    vmx = fmaxf(vmx, dpp<kRowRor2>(vmx));
    vmx = fmaxf(vmx, dpp<kRowRor4>(vmx));
    vmx = fmaxf(vmx, row_ror8(vmx));
    vmx = row_max(vmx);
    if (lane == 0) sm.vmax[wave] = vmx;
#pragma unroll
    for (int g = 0; g < 4; ++g) sm.vs[tid >> 5][(tid >> 3) & 3][g][tid & 7] = as_f32(r.sv[g]);
  }
}

// Precompute q~ for a staged tile and attend its 256 tokens.  Must follow
// stage_tile and a barrier.
__device__ __forceinline__ void attend_tile(Smem& sm, int tile0, int t_end, const float qv[16],
                                            const CodeConsts& cc_consts, int& sv_cur,
                                            WaveState& st) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int q = lane >> 4;

  // One exponent Sv for the tile's V scales (p~ = p * sV * 2^Sv); re-express
  // the running value sums when it changes.
  const int sv_new = prescale_exp(fmaxf(fmaxf(sm.vmax[0], sm.vmax[1]),
                                        fmaxf(sm.vmax[2], sm.vmax[3])));
  if (sv_new != sv_cur) {
    if (st.live) {
      const float t = __builtin_ldexpf(1.0f, sv_new - sv_cur);
      const f32x4 tv = {t, t, t, t};
      scale_acc(st, tv);
    }
    sv_cur = sv_new;
  }

  // ---- q~ = q * qscale * sK[d][G] as fp16 hi/lo (prescaled per group and
  // row) -----------------------------------------------------------------
  {
    const int gq = tid >> 5, rq = (tid >> 3) & 3, ksq = (tid >> 1) & 3, kbq = (tid & 1) * 2;
    const int d0 = ksq * 32 + kbq * 8;
    float x[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] = qv[i] * sm.ks[gq][d0 + i];
      amax = fmaxf(amax, fabsf(x[i]));
    }
    // max over the 8 consecutive lanes that share (group, row)
    amax = fmaxf(amax, dpp<kQuadXor1>(amax));
    amax = fmaxf(amax, dpp<kQuadXor2>(amax));
    amax = fmaxf(amax, dpp<kRowHalfMirror>(amax));
    const int sq = prescale_exp(amax);
    // channel d0 + 8h + kSlotByte[j] goes to k-slot j of k-block kbq + h
    float xs[16];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[8 * h + j] = __builtin_ldexpf(x[8 * h + kSlotByte[j]], sq);
    half8_t h0, l0, h1, l1;
    split_hilo(xs, h0, l0);
    split_hilo(xs + 8, h1, l1);
    *reinterpret_cast<half8_t*>(&sm.qt[gq][ksq][0][rq][kbq][0]) = h0;
    *reinterpret_cast<half8_t*>(&sm.qt[gq][ksq][0][rq][kbq + 1][0]) = h1;
    *reinterpret_cast<half8_t*>(&sm.qt[gq][ksq][1][rq][kbq][0]) = l0;
    *reinterpret_cast<half8_t*>(&sm.qt[gq][ksq][1][rq][kbq + 1][0]) = l1;
    if ((tid & 7) == 0) sm.qunscale[gq][rq] = __builtin_ldexpf(1.0f, -sq);
  }
  __syncthreads();

  // ---- each wave: one 64-token block = two 32-token chunks --------------
  // The two chunks are scored, folded into (m, z) and applied to u as one
  // block: independent MFMA chains, one max/sum reduction, one rescale.
  const int c0 = wave * 2;
  const int tok0 = tile0 + c0 * 32;
  if (tok0 < t_end) {  // wave-uniform
    const bool two = tok0 + 32 < t_end;  // the second chunk holds a real token
    const int part = n >> 3, row = n & 3;

    // S^T = codes^T * q~^T over 4 k-steps of 32 channels, both chunks
    const f32x4 zero_acc = {0.f, 0.f, 0.f, 0.f};
    f32x4 se[2] = {zero_acc, zero_acc}, so[2] = {zero_acc, zero_acc};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int d = ks * 32 + q * 8 + (n >> 1);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int c = c0 + cc;
        const i32x2 w = lds_tr8(&sm.big.codes.k[d * kKRow + c * 16 + (n & 1) * 8]);
        half8_t alo, ahi;
        codes_to_half(w, cc_consts, alo, ahi);
        const half8_t b = *reinterpret_cast<const half8_t*>(&sm.qt[c][ks][part][row][q][0]);
        se[cc] = mfma(alo, b, se[cc]);
        so[cc] = mfma(ahi, b, so[cc]);
      }
    }
    // hi + lo columns (still in units of 2^S of the chunk's group)
    float raw[2][8];  // [chunk][token 8q + t]
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        raw[cc][2 * i] = se[cc][i] + row_ror8(se[cc][i]);
        raw[cc][2 * i + 1] = so[cc][i] + row_ror8(so[cc][i]);
      }
    if (tok0 + 64 > t_end) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (tok0 + cc * 32 + 8 * q + t >= t_end) raw[cc][t] = -INFINITY;
    }

    // online softmax for row (n & 3); the prescale 2^-S > 0 commutes with max
    const float us0 = sm.qunscale[c0][row], us1 = sm.qunscale[c0 + 1][row];
    float mx0 = raw[0][0], mx1 = raw[1][0];
#pragma unroll
    for (int t = 1; t < 8; ++t) {
      mx0 = fmaxf(mx0, raw[0][t]);
      mx1 = fmaxf(mx1, raw[1][t]);
    }
    const float mx = row_max(fmaxf(mx0 * us0, mx1 * us1));
    const float m_new = fmaxf(st.m_run, mx);  // finite: the block has a real token
    const float alpha = fast_exp2(st.m_run - m_new);
    // pt = p * 2^Sv (the V-scale prescale rides in the exponent)
    const float shift = static_cast<float>(sv_cur) - m_new;
    float pt[2][8], psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      pt[0][t] = fast_exp2(fmaf(raw[0][t], us0, shift));
      pt[1][t] = fast_exp2(fmaf(raw[1][t], us1, shift));
      psum += pt[0][t] + pt[1][t];
    }
    psum = row_sum(psum) * __builtin_ldexpf(1.0f, -sv_cur);
    st.z_run = fmaf(alpha, st.z_run, psum);
    st.m_run = m_new;

    // rescale u by alpha of rows 0..3 (nothing to rescale before the first
    // block; skipped when no row's max moved)
    if (st.live) {
      const float a0 = as_f32(__builtin_amdgcn_readlane(static_cast<int>(as_u32(alpha)), 0));
      const float a1 = as_f32(__builtin_amdgcn_readlane(static_cast<int>(as_u32(alpha)), 1));
      const float a2 = as_f32(__builtin_amdgcn_readlane(static_cast<int>(as_u32(alpha)), 2));
      const float a3 = as_f32(__builtin_amdgcn_readlane(static_cast<int>(as_u32(alpha)), 3));
      if (!(a0 == 1.0f && a1 == 1.0f && a2 == 1.0f && a3 == 1.0f)) {
        const f32x4 av = {a0, a1, a2, a3};
        scale_acc(st, av);
      }
    }
    st.live = true;

    // p~ = (p 2^Sv) * sV[token][G'] for this lane's value group G' = n >> 2
    half8_t ah[2], al[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(&sm.vs[c0 + cc][q][n >> 2][0]);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(&sm.vs[c0 + cc][q][n >> 2][4]);
      float xt[8], xv[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        xt[t] = pt[cc][t] * v0[t];
        xt[t + 4] = pt[cc][t + 4] * v1[t];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) xv[j] = xt[kSlotByte[j]];  // token order -> k-slot order
      split_hilo(xv, ah[cc], al[cc]);
    }

    // u[4G'+r][f] += p~ x V codes, one feature group of 32 at a time
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        if (cc == 1 && !two) break;
        const int tok = (c0 + cc) * 32 + q * 8 + (n >> 1);
        const i32x2 w = lds_tr8(&sm.big.codes.v[tok * kVRow + g * 16 + (n & 1) * 8]);
        half8_t be, bo;
        codes_to_half(w, cc_consts, be, bo);
        st.acc[g][0] = mfma(ah[cc], be, st.acc[g][0]);
        st.acc[g][0] = mfma(al[cc], be, st.acc[g][0]);
        st.acc[g][1] = mfma(ah[cc], bo, st.acc[g][1]);
        st.acc[g][1] = mfma(al[cc], bo, st.acc[g][1]);
      }
    }
  }
  __syncthreads();  // before the next tile overwrites LDS
}

__global__ __launch_bounds__(kThreads) void attend_mfma_r4_kernel(AttendProblem p) {
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;  // MFMA column / A row
  const int q = lane >> 4;  // MFMA k-block / output row quad

  // Workgroup -> (KV head, split).  Workgroups are dealt to the 8 XCDs
  // round-robin; keep all splits of a head on one XCD so the head's partials
  // stay in that XCD's L2 for the combine.
  const int heads = p.B * p.Hkv;
  const int L = blockIdx.x;
  int head, split;
  if (heads % 8 == 0) {
    const int slot = L >> 3;
    head = (L & 7) + 8 * (slot / p.splits);
    split = slot % p.splits;
  } else {
    head = L / p.splits;
    split = L % p.splits;
  }
  const long long bh = head;
  const int rows = p.rows;
  Head h;
  h.N = p.N;
  h.npad = (p.N + 31) & ~31;
  h.ngroups = h.npad >> 5;
  h.krow_bytes = h.npad >> 1;
  h.kc = p.k_codes + bh * kD * h.krow_bytes;
  h.ksc = p.k_scales + bh * kD * h.ngroups;
  h.vc = p.v_codes + bh * static_cast<long long>(p.N) * (kD / 2);
  h.vsc = p.v_scales + bh * static_cast<long long>(p.N) * (kD / 32);

  const int t_begin = split * p.tokens_per_split;
  const int t_end = min(p.N, t_begin + p.tokens_per_split);

  // First tile's loads go out before anything else.
  TileRegs rt;
  if (t_begin < t_end) load_tile(h, t_begin, tid, rt);

  // q * qscale for this thread's q~ precompute slot (group tid>>5 varies per
  // tile; row (tid>>3)&3 and channels d0..d0+15 are fixed).  Rows past
  // `rows` read row 0 and are zeroed.
  float qv[16];
  {
    const int rq = (tid >> 3) & 3;
    const int d0 = ((tid >> 1) & 3) * 32 + (tid & 1) * 16;
    const float* qrow = p.q + (bh * rows + (rq < rows ? rq : 0)) * kD + d0;
    const float qs = rq < rows ? p.qscale : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(qrow + 4 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) qv[4 * i + j] = v[j] * qs;
    }
  }

  const CodeConsts cc_consts = code_consts();
  WaveState st;
  st.m_run = -INFINITY;
  st.z_run = 0.0f;
  st.live = false;
  {
    const f32x4 zero_acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 4; ++g) st.acc[g][0] = st.acc[g][1] = zero_acc;
  }
  int sv_cur = 0;  // exponent Sv the value sums are currently expressed in

  // Software pipeline: as soon as a tile sits in LDS its registers take the
  // next tile's loads, which stay in flight while this tile is attended.
  for (int tile0 = t_begin; tile0 < t_end; tile0 += kTile) {
    stage_tile(sm, rt);
    if (tile0 + kTile < t_end) load_tile(h, tile0 + kTile, tid, rt);
    __syncthreads();
    attend_tile(sm, tile0, t_end, qv, cc_consts, sv_cur, st);
  }

  // ---- this wave's u: lanes with q == G hold feature group G ----------------
  f32x4 ue = st.acc[0][0], uo = st.acc[0][1];
#pragma unroll
  for (int g = 1; g < 4; ++g) {
    if (q == g) {
      ue = st.acc[g][0];
      uo = st.acc[g][1];
    }
  }
  // acc rows are 4q + i = (value group q, query row i), in units of 2^Sv.
  const float fu = __builtin_ldexpf(1.0f, -sv_cur);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sm.big.wu[wave][i][q * 32 + 2 * n] = ue[i] * fu;
    sm.big.wu[wave][i][q * 32 + 2 * n + 1] = uo[i] * fu;
  }
  if (lane < 4) {
    sm.wm[wave][lane] = st.m_run;
    sm.wz[wave][lane] = st.z_run;
  }
  __syncthreads();

  // ---- merge the four waves: thread -> (row, two features) ---------------
  const int r = tid >> 6;          // 0..3
  const int f = (tid & 63) * 2;    // 0..126
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.wm[w][r]);
  float Z = 0.0f, U0 = 0.0f, U1 = 0.0f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.wm[w][r];
      if (mw == -INFINITY) continue;
      const float e = fast_exp2(mw - M);
      Z = fmaf(e, sm.wz[w][r], Z);
      U0 = fmaf(e, sm.big.wu[w][r][f], U0);
      U1 = fmaf(e, sm.big.wu[w][r][f + 1], U1);
    }
  }
  const long long row0 = bh * rows;
  if (p.splits == 1) {
    if (r < rows) {
      float* o = p.out + (row0 + r) * kD + f;
      o[0] = U0 / Z;
      o[1] = U1 / Z;
    }
    return;
  }

  // Fused combine: the last workgroup of this head to arrive merges all
  // splits.  Partials are written with device-scope stores (written through
  // to the device coherence point, so no cache flush is needed), each thread
  // waits for its stores to be acknowledged, and only then does thread 0
  // take a ticket.  The last arriver reads the partials with device-scope
  // loads.  (A device-scope release/acquire fence would instead write back
  // and invalidate the whole L2 of the XCD, once per workgroup.)
  const long long total_rows = static_cast<long long>(p.B) * p.Hkv * rows;
  if (r < rows) {
    const long long prow = split * total_rows + row0 + r;
    __hip_atomic_store(&p.part_u[prow * kD + f], U0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p.part_u[prow * kD + f + 1], U1, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (f == 0) {
      __hip_atomic_store(&p.part_m[prow], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.part_z[prow], Z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(&p.counters[bh], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sm.last = prev == static_cast<unsigned>(p.splits - 1);
  }
  __syncthreads();
  if (!sm.last) return;
  if (r < rows) {
    // Online merge over the splits, eight at a time so the loads of a batch
    // are all in flight together.
    const long long prow = row0 + r;
    float Mg = -INFINITY, Zg = 0.0f, V0 = 0.0f, V1 = 0.0f;
    for (int s0 = 0; s0 < p.splits; s0 += 8) {
      float ms[8], zs[8], u0[8], u1[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sidx = s0 + j < p.splits ? s0 + j : s0;
        const long long pr = sidx * total_rows + prow;
        ms[j] = __hip_atomic_load(&p.part_m[pr], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        zs[j] = __hip_atomic_load(&p.part_z[pr], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        u0[j] = __hip_atomic_load(&p.part_u[pr * kD + f], __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        u1[j] = __hip_atomic_load(&p.part_u[pr * kD + f + 1], __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        if (s0 + j >= p.splits) ms[j] = -INFINITY;
      }
      float mb = Mg;
#pragma unroll
      for (int j = 0; j < 8; ++j) mb = fmaxf(mb, ms[j]);
      if (mb == -INFINITY) continue;
      const float a = fast_exp2(Mg - mb);  // 0 while nothing merged yet
      Zg *= a;
      V0 *= a;
      V1 *= a;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (ms[j] == -INFINITY) continue;
        const float e = fast_exp2(ms[j] - mb);
        Zg = fmaf(e, zs[j], Zg);
        V0 = fmaf(e, u0[j], V0);
        V1 = fmaf(e, u1[j], V1);
      }
      Mg = mb;
    }
    float* o = p.out + prow * kD + f;
    o[0] = V0 / Zg;
    o[1] = V1 / Zg;
  }
  if (tid == 0) __hip_atomic_store(&p.counters[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

int mfma_tokens_per_split(int N, int splits) {
  const int per = (N + splits - 1) / splits;
  return (per + kTile - 1) / kTile * kTile;
}

hipError_t launch_attend_mfma(const AttendProblem& p, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(p.splits) * p.B * p.Hkv;
  hipLaunchKernelGGL(attend_mfma_r4_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvq
