// Matrix-core fused attention for the 4-bit, group-32, D=128 packed cache
// with at most 4 query rows per KV head (GQA group x queries <= 4).
//
// Method: the blocked online softmax of "Block KV decoding: less workspace,
// more time" (huhohoo.com/en/docs/llm/kv-block-decode-cost), section "Do not
// average independently normalized blocks", and of "给长前缀列一张有单位的资源账本"
// (codingai-lec05.pages.dev resource-ledger), section "why FlashAttention need
// not keep the whole heat map": per query row a reference max m, an
// exponential sum z and an unnormalized value sum u, both sums relative to
// 2^m and rescaled by 2^(m_old - m_new) whenever the reference moves.
// Scores are in base-2 units (q carries sm_scale * log2 e).  Waves and KV
// splits are merged with the same rescale ("two stops of the online
// accumulation" on the same page: partial statistics are composable).
//
// Lazy reference.  The reference moves only when a block's max exceeds it by
// more than kLazy (2^kLazy bounds every p = 2^(s - m) in between); the pages'
// recurrence moves it on every increase.  Both give the same u / z up to
// rounding (the rescale is exact algebra), and this one skips most rescales.
//
// Packed format ("KV分组打包：4-bit到底省了多少？", huhohoo.com/docs/llm/kv-packed-groups,
// "what a byte holds"), in the 32-token block byte order of kvq_layout.h,
// which puts each lane's matrix-core operand bytes at consecutive addresses:
//   K block (2 KB): lane l = 16 q + n reads 8 bytes at ks*512 + 8 l =
//     channels ks*32 + 8q + (0..7) of token pair n (tokens 2n low nibble,
//     2n+1 high nibble), k-step ks = 0..3;
//   V block (2 KB): lane (n, q) reads 8 bytes at q*512 + g*128 + 8n =
//     tokens 8q + (0..7) of byte column 16g + n (features 32g + 2n, +1);
//   K scales of the block's group: 128 floats, channel order;
//   V scales of the block: [value group][32 tokens].
// Every load is a contiguous, coalesced global load into VGPRs; no LDS
// staging, no barriers in the main loop.  Each wave streams its own blocks
// and keeps the next block's loads in flight while it computes one.
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
// each set is multiplied by a power of two that keeps its largest element
// inside the fp16 range and the lo halves of all elements that matter out of
// the subnormal range; the factor is exact and divided out in float32.
//
// Math per 32-token block, one wave:
//   S^T[pair][col] = codes^T (A: 16 token pairs x 32 channels per k-step,
//     low and high nibbles as two products) x q~^T (B: 32 channels x 16
//     columns; column n = (hi|lo part n >> 3, query row n & 3));
//   u[4 G' + r][f] += p~_G' (A: 16 rows = 4 value groups x 4 query rows)
//     x V codes (B: 32 tokens x 16 feature pairs).
// The A-row layout 4 G' + r lets every lane form the p~ of one value group
// only; rows whose group differs from the B columns' group are discarded.
#include "kvq_internal.h"
#include "kvq_layout.h"
#include "kvq_mfma_common.h"

namespace kvq {
namespace {

#ifndef KVQ_MFMA_WAVES
#define KVQ_MFMA_WAVES 8
#endif
constexpr int kWaves = KVQ_MFMA_WAVES;   // waves per workgroup, one KV head split each
constexpr int kThreads = kWaves * 64;
constexpr int kOut = 4 * 128;            // outputs of one KV head: 4 rows x D
constexpr int kSlots = kOut / kThreads > 0 ? kOut / kThreads : 1;  // outputs per thread
constexpr int kD = 128;
constexpr int kBlockBytes = 2048;   // K or V codes of one 32-token block
constexpr int kBlockScales = 128;   // K or V scales of one block
constexpr float kLazy = 6.0f;       // reference moves only past m + kLazy
// V prescale: max V scale * 2^Sv is set to [2^8, 2^9) and kept while it
// stays in [2^2, 2^9): with p <= 2^kLazy, p~ < 2^15 fits fp16.
constexpr int kSvTop = 9;
constexpr int kSvLow = 2;

struct alignas(16) Smem {
  union {
    _Float16 qt[kWaves][4][2][4][4][8];  // per wave: q~ [kstep][hi|lo][row][kblock][8]
    float wu[kWaves][4][kD];             // per-wave u for the final merge
  } u;
  float qus[kWaves][4];                  // 2^-S of q~ per row
  float qs[4][kD];                       // q * qscale, the workgroup's query rows
  float wm[kWaves][4];
  float wz[kWaves][4];
  int last;
};

// One block's operands, as loaded by one lane.
struct BlockRegs {
  i32x2 k[4];   // K codes, k-step 0..3
  i32x2 v[4];   // V codes, feature group 0..3
  f32x4 ks[2];  // K scales of channels d0 .. d0+7 (precompute slot)
  f32x4 vs[2];  // V scales of value group n >> 2, tokens 8q .. 8q+7
};

struct Head {
  const uint8_t* kc;
  const float* ksc;
  const uint8_t* vc;
  const float* vsc;
};

// Loaders of the four parts of one block's operands.  Each part is
// reloaded for the next block as soon as the current block has consumed it,
// so about one block of loads stays in flight with a single register set.
struct Lanes {
  unsigned k_off, v_off, ks_off, vs_off;  // byte / element offsets of this lane
};
__device__ __forceinline__ Lanes lane_offsets(int lane, int d0) {
  const int n = lane & 15, q = lane >> 4;
  return {static_cast<unsigned>(lane * 8), static_cast<unsigned>(q * 512 + n * 8),
          static_cast<unsigned>(d0), static_cast<unsigned>((n >> 2) * 32 + q * 8)};
}
__device__ __forceinline__ void load_ks(BlockRegs& r, const Head& h, int blk, const Lanes& o) {
  const float* p = h.ksc + static_cast<long long>(blk) * kBlockScales + o.ks_off;
  r.ks[0] = *reinterpret_cast<const f32x4*>(p);
  r.ks[1] = *reinterpret_cast<const f32x4*>(p + 4);
}
__device__ __forceinline__ void load_k(BlockRegs& r, const Head& h, int blk, const Lanes& o) {
  const uint8_t* p = h.kc + static_cast<long long>(blk) * kBlockBytes + o.k_off;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.k[i] = *reinterpret_cast<const i32x2*>(p + i * 512);
}
__device__ __forceinline__ void load_vs(BlockRegs& r, const Head& h, int blk, const Lanes& o) {
  const float* p = h.vsc + static_cast<long long>(blk) * kBlockScales + o.vs_off;
  r.vs[0] = *reinterpret_cast<const f32x4*>(p);
  r.vs[1] = *reinterpret_cast<const f32x4*>(p + 4);
}
__device__ __forceinline__ void load_v(BlockRegs& r, const Head& h, int blk, const Lanes& o) {
  const uint8_t* p = h.vc + static_cast<long long>(blk) * kBlockBytes + o.v_off;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.v[i] = *reinterpret_cast<const i32x2*>(p + i * 128);
}
__device__ __forceinline__ void load_block(BlockRegs& r, const Head& h, int blk, const Lanes& o) {
  load_ks(r, h, blk, o);
  load_k(r, h, blk, o);
  load_vs(r, h, blk, o);
  load_v(r, h, blk, o);
}

// Running state of one wave.  Lane (n, q) tracks query row n & 3: m is the
// row's reference max (the same in all its lanes), z the sum of p over this
// lane's tokens (8q .. 8q+7 of each block; summed over the q-blocks at the
// end).  acc[g][e] holds the value sums of feature group g, even (e = 0) or
// odd (e = 1) features, rows 4q + i = (value group q, query row i), in
// units of 2^(m + sv).  vhi / vlo are the V-scale bounds 2^(kSvTop - sv)
// and 2^(kSvLow - sv) that keep the current sv valid.
struct WaveState {
  float m, z;
  f32x4 acc[4][2];
  int sv;
  float vhi, vlo;
  bool live;  // a block has been folded in
};

// Attend one 32-token block (tokens tok0 .. tok0+31; with kMasked, those
// >= t_end are masked out).
template <bool kMasked>
__device__ __forceinline__ void attend_block(Smem& sm, BlockRegs& br, int tok0, int t_end,
                                             const CodeConsts& cc, WaveState& ws, const Head& h,
                                             int next, const Lanes& lo_) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int q = lane >> 4;

  // q~ of this block's K group: lane (rq, ksq, kbq) = (lane >> 4, (lane >> 2)
  // & 3, lane & 3) forms channels ksq*32 + kbq*8 .. +7 of row rq, prescaled
  // per row (the 16 lanes of a row are one DPP row), and parks hi / lo in
  // this wave's LDS slots in the B-operand order.
  {
    const int rq = lane >> 4, ksq = (lane >> 2) & 3, kbq = lane & 3;
    const f32x4 qa = *reinterpret_cast<const f32x4*>(&sm.qs[rq][ksq * 32 + kbq * 8]);
    const f32x4 qb = *reinterpret_cast<const f32x4*>(&sm.qs[rq][ksq * 32 + kbq * 8 + 4]);
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = qa[i] * br.ks[0][i];
      x[i + 4] = qb[i] * br.ks[1][i];
    }
    float amax = fmaxf(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))),
                       fmaxf(fmaxf(fabsf(x[4]), fabsf(x[5])), fmaxf(fabsf(x[6]), fabsf(x[7]))));
    amax = fmaxf(amax, dpp<kRowRor1>(amax));
    amax = fmaxf(amax, dpp<kRowRor2>(amax));
    amax = fmaxf(amax, dpp<kRowRor4>(amax));
    amax = fmaxf(amax, dpp<kRowRor8>(amax));
    const int sq = prescale_exp(amax, 15);
    float xs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[j] = __builtin_ldexpf(x[kSlotByte[j]], sq);
    half8_t hi, lo;
    split_hilo(xs, hi, lo);
    *reinterpret_cast<half8_t*>(&sm.u.qt[wave][ksq][0][rq][kbq][0]) = hi;
    *reinterpret_cast<half8_t*>(&sm.u.qt[wave][ksq][1][rq][kbq][0]) = lo;
    if ((lane & 15) == 0) sm.qus[wave][rq] = __builtin_ldexpf(1.0f, -sq);
  }
  load_ks(br, h, next, lo_);

  // S^T = codes^T * q~^T over 4 k-steps of 32 channels.
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 se = zero4, so = zero4;
  const int part = n >> 3, row = n & 3;
  const uint8_t* knext = h.kc + static_cast<long long>(next) * kBlockBytes + lo_.k_off;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    half8_t alo, ahi;
    codes_to_half(br.k[ks], cc, alo, ahi);
    br.k[ks] = *reinterpret_cast<const i32x2*>(knext + ks * 512);  // next block's k-step
    const half8_t b = *reinterpret_cast<const half8_t*>(&sm.u.qt[wave][ks][part][row][q][0]);
    se = mfma(alo, b, se);
    so = mfma(ahi, b, so);
  }
  const float us = sm.qus[wave][row];
  // hi + lo columns: token 8q + t in raw[t], in units of 2^S of q~
  float raw[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    raw[2 * i] = se[i] + dpp<kRowRor8>(se[i]);
    raw[2 * i + 1] = so[i] + dpp<kRowRor8>(so[i]);
  }
  if (kMasked) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (tok0 + 8 * q + t >= t_end) raw[t] = -INFINITY;
  }
  // this lane's max over its 8 tokens, base-2 units (2^-S > 0 commutes with max)
  const float lmx =
      fmaxf(fmaxf(fmaxf(raw[0], raw[1]), fmaxf(raw[2], raw[3])),
            fmaxf(fmaxf(raw[4], raw[5]), fmaxf(raw[6], raw[7]))) * us;
  // this lane's largest V scale (value group n >> 2, tokens 8q .. 8q+7)
  const float lvs = fmaxf(fmaxf(fmaxf(br.vs[0][0], br.vs[0][1]), fmaxf(br.vs[0][2], br.vs[0][3])),
                          fmaxf(fmaxf(br.vs[1][0], br.vs[1][1]), fmaxf(br.vs[1][2], br.vs[1][3])));

  // Move the reference when any row's block max overshoots it by more than
  // kLazy, the V prescale when the block's largest V scale leaves
  // [2^kSvLow, 2^kSvTop) after scaling; both decisions are wave-uniform.
  const bool move_m = !ws.live || __builtin_amdgcn_ballot_w64(lmx > ws.m + kLazy) != 0;
  const bool move_sv = !ws.live || __builtin_amdgcn_ballot_w64(!(lvs < ws.vhi)) != 0 ||
                       __builtin_amdgcn_ballot_w64(lvs >= ws.vlo) == 0;
  if (move_m || move_sv) {
    const float mx = qblock_max(lmx);  // row max over the block; finite
    float vmx = fmaxf(lvs, dpp<kRowRor4>(lvs));
    vmx = qblock_max(fmaxf(vmx, dpp<kRowRor8>(vmx)));  // block max over the wave
    const float m_new = ws.live ? (mx > ws.m + kLazy ? mx : ws.m) : mx;
    const int sv_new = move_sv ? prescale_exp(vmx, kSvTop) : ws.sv;
    if (ws.live) {
      const float alpha = fast_exp2(ws.m - m_new);
      ws.z *= alpha;
      const float t = __builtin_ldexpf(1.0f, sv_new - ws.sv);
      const float a0 = as_f32(__builtin_amdgcn_readlane(static_cast<int>(as_u32(alpha)), 0));
      const float a1 = as_f32(__builtin_amdgcn_readlane(static_cast<int>(as_u32(alpha)), 1));
      const float a2 = as_f32(__builtin_amdgcn_readlane(static_cast<int>(as_u32(alpha)), 2));
      const float a3 = as_f32(__builtin_amdgcn_readlane(static_cast<int>(as_u32(alpha)), 3));
      const f32x4 f = {a0 * t, a1 * t, a2 * t, a3 * t};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        ws.acc[g][0] *= f;
        ws.acc[g][1] *= f;
      }
    }
    ws.m = m_new;
    ws.sv = sv_new;
    ws.vhi = __builtin_ldexpf(1.0f, kSvTop - sv_new);
    ws.vlo = __builtin_ldexpf(1.0f, kSvLow - sv_new);
    ws.live = true;
  }

  // pt = 2^(s - m + Sv) (the V prescale rides in the exponent), z += sum p
  const float shift = static_cast<float>(ws.sv) - ws.m;
  float pt[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) pt[t] = fast_exp2(fmaf(raw[t], us, shift));
  const float psum = ((pt[0] + pt[1]) + (pt[2] + pt[3])) + ((pt[4] + pt[5]) + (pt[6] + pt[7]));
  ws.z = fmaf(psum, __builtin_ldexpf(1.0f, -ws.sv), ws.z);

  // p~ = pt * sV[token][G'] for this lane's value group, in k-slot order
  half8_t ah, al;
  {
    float xt[8], xv[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      xt[t] = pt[t] * br.vs[0][t];
      xt[t + 4] = pt[t + 4] * br.vs[1][t];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = xt[kSlotByte[j]];
    split_hilo(xv, ah, al);
  }
  load_vs(br, h, next, lo_);

  // u[4G'+r][f] += p~ x V codes, one feature group of 32 at a time
  const uint8_t* vnext = h.vc + static_cast<long long>(next) * kBlockBytes + lo_.v_off;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    half8_t be, bo;
    codes_to_half(br.v[g], cc, be, bo);
    br.v[g] = *reinterpret_cast<const i32x2*>(vnext + g * 128);  // next block's group
    ws.acc[g][0] = mfma(ah, be, ws.acc[g][0]);
    ws.acc[g][0] = mfma(al, be, ws.acc[g][0]);
    ws.acc[g][1] = mfma(ah, bo, ws.acc[g][1]);
    ws.acc[g][1] = mfma(al, bo, ws.acc[g][1]);
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void
attend_mfma_r4_kernel(AttendProblem p) {
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int nblocks = (p.N + kBlockTokens - 1) / kBlockTokens;
  Head h;
  h.kc = p.k_codes + bh * nblocks * kBlockBytes;
  h.ksc = p.k_scales + bh * nblocks * kBlockScales;
  h.vc = p.v_codes + bh * nblocks * kBlockBytes;
  h.vsc = p.v_scales + bh * nblocks * kBlockScales;

  const int t_begin = split * p.tokens_per_split;
  const int t_end = min(p.N, t_begin + p.tokens_per_split);
  // blocks of this split: [b_begin, b_end); wave w takes b_begin + w + 4i
  const int b_begin = t_begin / kBlockTokens;
  const int b_end = t_end > t_begin ? (t_end + kBlockTokens - 1) / kBlockTokens : b_begin;
  const int b_first = b_begin + wave;
  const int b_last = b_first + (b_end - 1 - b_first) / kWaves * kWaves;  // valid if b_first < b_end

  // this lane's K-scale slot in the q~ precompute: channels d0 .. d0+7
  const int d0 = ((lane >> 2) & 3) * 32 + (lane & 3) * 8;
  const Lanes lo = lane_offsets(lane, d0);

  // The block holding token N-1 is masked when N is not a multiple of 32;
  // the wave that owns it attends it first, so only the peeled first block
  // carries masking code.  Its loads go out before the query is staged.
  const bool active = b_first < b_end;  // wave-uniform
  const bool partial = (p.N % kBlockTokens) != 0 && b_last == nblocks - 1;
  const int first = partial ? b_last : b_first;
  const int loop_begin = partial ? b_first : b_first + kWaves;
  const int loop_end = partial ? b_last - kWaves : b_last;  // inclusive
  BlockRegs br;
  if (active) load_block(br, h, first, lo);

  // q * qscale of the head's query rows into LDS, output slot e = tid +
  // j * kThreads -> (row e >> 7, channel e & 127).  Rows past `rows` are zero.
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int e = tid + j * kThreads;
    if (e < kOut) {
      const int rq = e >> 7, c = e & 127;
      sm.qs[rq][c] = rq < rows ? p.q[(bh * rows + rq) * kD + c] * p.qscale : 0.0f;
    }
  }
  __syncthreads();

  const CodeConsts cc = code_consts();
  WaveState ws;
  ws.m = -INFINITY;
  ws.z = 0.0f;
  ws.sv = 0;
  ws.vhi = ws.vlo = 0.0f;
  ws.live = false;
  {
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 4; ++g) ws.acc[g][0] = ws.acc[g][1] = zero4;
  }

  if (active) {
    // One register set: each part of the next block is loaded as soon as
    // the current block has consumed that part.
    attend_block<true>(sm, br, first * kBlockTokens, t_end, cc, ws, h,
                       loop_begin <= loop_end ? loop_begin : first, lo);
    for (int b = loop_begin; b <= loop_end; b += kWaves)
      attend_block<false>(sm, br, b * kBlockTokens, t_end, cc, ws, h, min(b + kWaves, loop_end),
                          lo);
  }
  // z of each row: sum this lane's share over the four q-blocks
  ws.z = qblock_sum(ws.z);

  // ---- this wave's u: lanes with q == G hold feature group G ----------------
  f32x4 ue = ws.acc[0][0], uo = ws.acc[0][1];
#pragma unroll
  for (int g = 1; g < 4; ++g) {
    if (q == g) {
      ue = ws.acc[g][0];
      uo = ws.acc[g][1];
    }
  }
  __syncthreads();  // every wave is done with its q~ slots (aliased by wu)
  const float fu = __builtin_ldexpf(1.0f, -ws.sv);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sm.u.wu[wave][i][q * 32 + 2 * n] = ue[i] * fu;
    sm.u.wu[wave][i][q * 32 + 2 * n + 1] = uo[i] * fu;
  }
  if (lane < 4) {
    sm.wm[wave][lane] = ws.m;
    sm.wz[wave][lane] = ws.z;
  }
  __syncthreads();

  // ---- merge the waves: thread -> row r, features f0 .. f0 + kSlots - 1 ----
  const int e0 = tid * kSlots;
  const int r = e0 >> 7, f0 = e0 & 127;
  float M = -INFINITY, Z = 0.0f, U[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) U[j] = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.wm[w][r]);
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.wm[w][r];
      if (mw == -INFINITY) continue;
      const float x = fast_exp2(mw - M);
      Z = fmaf(x, sm.wz[w][r], Z);
#pragma unroll
      for (int j = 0; j < kSlots; ++j) U[j] = fmaf(x, sm.u.wu[w][r][f0 + j], U[j]);
    }
  }
  if (p.splits == 1) {
    if (r < rows) {
#pragma unroll
      for (int j = 0; j < kSlots; ++j) p.out[(bh * rows + r) * kD + f0 + j] = U[j] / Z;
    }
    return;
  }
  split_combine<kSlots, kSlots, 0>(p, split, bh, r, f0, U, M, Z, &sm.last);
}

}  // namespace

int mfma_tokens_per_split(int N, int splits) {
  const int per = (N + splits - 1) / splits;
  return (per + kBlockTokens - 1) / kBlockTokens * kBlockTokens;
}

hipError_t launch_attend_mfma(const AttendProblem& p, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(p.splits) * p.B * p.Hkv;
  hipLaunchKernelGGL(attend_mfma_r4_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvq
